// tq_decode_attn_append_noalloc: the one-launch decode step of tq_decode_attn_append with its
// scratch (per-(batch, kv head) arrival counters and the per-split partials) in a file-scope
// device array instead of a caller workspace, so the call allocates nothing.
//
// Scratch map (bytes; one copy per GPU, held until the process ends):
//   [0, kCounterBytes)            arrival counters, one u32 per (batch, kv head).  Nothing else is
//                                 ever written here and every completed call leaves its counters
//                                 at zero, so they are zero at the start of every call on the GPU
//                                 once the first call has cleared the region.
//   [kCounterBytes, kScratchBytes) the call's partials (m, l) and rotated-domain sums per
//                                 (batch, query head, split), laid out as in the workspace.
// Calls that overlap in time on one GPU share this memory and race: order them on one stream
// (or with events).
#include <mutex>

#include "tq_launch.h"

namespace tq {
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr size_t kCounterBytes = size_t(64) << 10;
constexpr int kMaxUnits = int(kCounterBytes / sizeof(unsigned));  // batch * n_kv_heads
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on each GPU (the host-side name is only a stand-in for it), and
// whether its counter region has been cleared on that GPU.
struct ScratchSlot {
  uint8_t *ptr;
  bool cleared;
};
std::mutex g_mutex;
ScratchSlot g_slots[kMaxDevices];

__global__ void clear_counters(unsigned *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The current GPU's scratch; on the first call on a GPU, looks up the array's address there and
// clears the counter region with a kernel on `stream` (a fill kernel rather than a memset, so a
// captured first call replays correctly).  Returns a tq_status.
int device_scratch(hipStream_t stream, uint8_t **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  ScratchSlot &slot = g_slots[dev];
  if (slot.ptr == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TQ_ERR_HIP;
    slot.ptr = static_cast<uint8_t *>(p);
  }
  if (!slot.cleared) {
    clear_counters<<<(kMaxUnits + 255) / 256, 256, 0, stream>>>(reinterpret_cast<unsigned *>(slot.ptr), kMaxUnits);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
    slot.cleared = true;
  }
  *out = slot.ptr;
  return TQ_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace
}  // namespace tq

using namespace tq;

extern "C" int tq_decode_attn_append_noalloc(const tq_cache *k, const tq_cache *v, const void *xk, const void *xv,
                                             int x_dtype, const void *q, int q_dtype, int n_q_heads,
                                             const int32_t *seq_lens, int ctx_len, float scale, float *out,
                                             float *lse, void *hip_stream) {
  DecodeArgs a{};
  WorkspaceLayout w{};
  const int st = setup_decode_append(k, v, xk, xv, x_dtype, q, q_dtype, n_q_heads, seq_lens, ctx_len, scale, out,
                                     lse, a, w);
  if (st != TQ_OK) return st;
  // the one-launch path only: other code widths need the two-launch path and its workspace
  if (!decode_fused_shape_ok(a)) return TQ_ERR_UNSUPPORTED;
  // sizes, checked before any HIP call: counters of every (batch, kv head) in the counter
  // region, the partials in the rest
  const size_t rows = (size_t)a.batch * a.n_q_heads * a.fplan.n_splits;
  const size_t ml_bytes = align256(rows * sizeof(float2));
  const size_t o_bytes = align256(rows * kD * sizeof(float));
  if ((long)a.batch * a.n_kv_heads > kMaxUnits || kCounterBytes + ml_bytes + o_bytes > kScratchBytes)
    return TQ_ERR_WORKSPACE;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  uint8_t *base = nullptr;
  const int sst = device_scratch(stream, &base);
  if (sst != TQ_OK) return sst;
  a.counters = reinterpret_cast<unsigned *>(base);
  a.fpart_ml = reinterpret_cast<float2 *>(base + kCounterBytes);
  a.fpart_o = reinterpret_cast<float *>(base + kCounterBytes + ml_bytes);
  a.xk = xk;
  a.xv = xv;
  a.x_dtype = x_dtype;
  return launch_decode_fused(a, compute_units(), stream) == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

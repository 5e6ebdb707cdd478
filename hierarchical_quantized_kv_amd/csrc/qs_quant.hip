// qs_quant.hip -- launchers of the append, flush, prefill and device-state kernels, and the
// work-item slots of the attention kernels (their occupancy on the current device).
#include <atomic>

#include "qs_device.h"

namespace qs {

// ------------------------------------------------------------------------------------------
// Device-mode commit: the pending operations of a layer, then for a flush its counter update.
// Runs after every kernel that read the old counters (stream order); the same checks as the
// host verbs decide, and a failing operation leaves the counters and sets its error bit.
// ------------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void state_kernel(const StateArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.nl * a.B) return;
  const int b = idx % a.B, layer = a.l0 + idx / a.B;
  int32_t* st = a.state + ((size_t)layer * a.B + b) * kStateInts;
  int32_t bad = 0;
  int nq = st[0], head = st[2];
  int nt = apply_pending(st[1], a.pend, b, &bad);
  if (a.op == 1 && nt >= a.thr) {
    if (nq + a.G <= a.T) {
      nq += a.G;
      nt -= a.G;
      head ^= a.G;
    } else {
      bad |= kDevErrFlush;
    }
  }
  st[0] = nq;
  st[1] = nt;
  st[2] = head;
  if (bad) atomicOr(a.err, bad);
}

template <int D, int NB>
void launch_append_n(const AppendArgs& f, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((append_kernel<D, NB>), grid, dim3(256), 0, st, narrow<NB>(f));
}

template <int D>
void launch_append_d(const AppendArgs& a, dim3 grid, hipStream_t st) {
  switch (batch_bucket(a.B)) {
    case 1: launch_append_n<D, 1>(a, grid, st); break;
    case 8: launch_append_n<D, 8>(a, grid, st); break;
    default: launch_append_n<D, QS_MAX_BATCH>(a, grid, st); break;
  }
}

hipError_t launch_append(const AppendArgs& a, int D, hipStream_t st) {
  const long long rows = (long long)a.B * a.n_rows * a.H;
  const long long threads = rows * (D / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (D == 128) launch_append_d<128>(a, grid, st);
  else launch_append_d<64>(a, grid, st);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int D, int max_groups, hipStream_t st) {
  const int rows = max_groups + (a.rest_row >= 0 ? 1 : 0);
  if (rows <= 0) return hipSuccess;
  const dim3 grid(a.H * 2, rows, a.B);  // per head: a key and a value workgroup
  if (D == 128) hipLaunchKernelGGL(prefill_kernel<128>, grid, dim3(64 * kQuantWaves), 0, st, a);
  else hipLaunchKernelGGL(prefill_kernel<64>, grid, dim3(64 * kQuantWaves), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_state(const StateArgs& a, hipStream_t st) {
  const int n = a.nl * a.B;
  hipLaunchKernelGGL(state_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_flush(const FlushArgs& a, int D, int n_layers, hipStream_t st) {
  const dim3 grid(a.H * 2, a.n_sel, n_layers);  // per head: a key and a value workgroup
  if (D == 128) hipLaunchKernelGGL(flush_kernel<128>, grid, dim3(64 * kQuantWaves), 0, st, a);
  else hipLaunchKernelGGL(flush_kernel<64>, grid, dim3(64 * kQuantWaves), 0, st, a);
  return hipGetLastError();
}

// Kernel of each attention mode (defined in that mode's translation unit).
const void* attn_fn_host(int D, bool draft, int bucket, bool meta16);
const void* attn_fn_dev(int D, bool draft, int bucket, bool meta16);
const void* attn_fn_app(int D, bool draft, int bucket, bool meta16);
const void* attn_fn_gqa(int D, bool draft, int bucket, bool meta16, bool pair);
const void* attn_fn_split_host(int D, bool draft, int bucket, int fmt);
const void* attn_fn_split_app(int D, bool draft, int bucket);
static const void* attn_fn_mode(int mode, int D, bool draft, int bucket, bool meta16, int fmt,
                                bool pair) {
  if (fmt != kFmtNibble)  // split-upper layout: host mode and fused append only
    return mode == kModeAppend ? attn_fn_split_app(D, draft, bucket)
                               : attn_fn_split_host(D, draft, bucket, fmt);
  switch (mode) {
    case kModeDev: return attn_fn_dev(D, draft, bucket, meta16);
    case kModeAppend: return attn_fn_app(D, draft, bucket, meta16);
    case kModeGqa: return attn_fn_gqa(D, draft, bucket, meta16, pair);
    default: return attn_fn_host(D, draft, bucket, meta16);
  }
}

// Work-item slots of one attention pass on the current device: compute units times the
// one-wave workgroups of that kernel a compute unit holds at once (cached per device).  pair:
// the grouped-query draft's paired form (gqa_paired).
int attention_slots(int D, bool draft, int B, int mode, bool meta16, int fmt, bool pair) {
  constexpr int kMaxDev = 64;
  // filled on first use; concurrent callers at worst compute the same value twice
  static std::atomic<int> cache[kMaxDev][3][2][2][2][4][3][2];
  int id = 0;
  if (hipGetDevice(&id) != hipSuccess || id < 0 || id >= kMaxDev || mode < 0 || mode > 3 ||
      fmt < 0 || fmt > 2)
    return 0;
  pair = pair && mode == kModeGqa && draft && fmt == kFmtNibble;
  const int bucket = batch_bucket(B);
  std::atomic<int>& slot =
      cache[id][fmt][meta16][D == 128][draft][mode][bucket == 1 ? 0 : (bucket == 8 ? 1 : 2)][pair];
  const int known = slot.load(std::memory_order_relaxed);
  if (known > 0) return known;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, id) != hipSuccess) return 0;
  const void* fn = attn_fn_mode(mode, D, draft, bucket, meta16, fmt, pair);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64, 0) != hipSuccess) return 0;
  const int n = cus * per_cu;
  slot.store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace qs

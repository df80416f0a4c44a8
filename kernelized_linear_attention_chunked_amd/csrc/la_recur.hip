// Whole-sequence token-by-token evaluation of the gated and delta recurrences
// (the LinearAttention operator page, ai.onnx since version 27, "Description":
// the recurrence is defined one token at a time), one workgroup per (batch, kv
// head) unit and query-head group, the state in registers from the first
// token to the last.  It serves fp32 inputs at head size 128 with a per-key-dim
// decay, whose fp32 chunk tiles and table of cumulative decays do not fit the
// LDS of the chunk kernels; one launch replaces a launch of the T == 1 step
// kernel per token (which read and wrote the whole state every token).
#include "la_launch.hpp"
#include "la_recur.hpp"

namespace la {

constexpr int kRecurThreads = 256;

template <typename IT, int D, int GW, int DK, bool DELTA>
__global__ __launch_bounds__(kRecurThreads) void recur_kernel(RecurArgs a) {
  constexpr int NTH = kRecurThreads;
  constexpr int HP = recur_heads<D, NTH, GW>(48 * 1024);
  static_assert(HP >= 1, "LDS");
  __shared__ __align__(16) unsigned char lds[recur_lds_bytes<D, NTH, GW, HP>()];
  const int hs = a.hsplit > 1 ? a.hsplit : 1;
  const int hg = blockIdx.x % hs;
  const int u = blockIdx.x / hs;
  const int b = u / a.Hkv, j = u % a.Hkv;
  const int64_t T = a.T;
  const int64_t QS = (int64_t)a.Hq * D, KS = (int64_t)a.Hkv * D;
  RecurPtrs rp;
  rp.q = (const IT*)a.q + b * T * QS + (int64_t)(j * GW * hs + hg * GW) * D;
  rp.out = (IT*)a.out + b * T * QS + (int64_t)(j * GW * hs + hg * GW) * D;
  rp.k = (const IT*)a.k + b * T * KS + (int64_t)j * D;
  rp.v = (const IT*)a.v + b * T * KS + (int64_t)j * D;
  rp.decay = DK == 2 ? (const void*)((const IT*)a.decay + b * T * KS + (int64_t)j * D)
                     : (DK == 1 ? (const void*)((const IT*)a.decay + b * T * a.Hkv + j) : nullptr);
  rp.beta = DELTA ? (const void*)((const IT*)a.beta + b * T * a.beta_heads + (a.beta_heads > 1 ? j : 0)) : nullptr;
  rp.s_in = a.s_in ? a.s_in + (int64_t)u * D * D : nullptr;
  rp.s_out = hg == 0 ? a.s_out + (int64_t)u * D * D : nullptr;
  rp.qs = QS;
  rp.ks = KS;
  rp.gs = DK == 2 ? KS : a.Hkv;
  rp.bs = a.beta_heads;
  rp.t0 = 0;
  rp.t1 = (int)T;
  rp.scale = a.scale;
  token_recurrence<IT, D, NTH, GW, HP, DK, DELTA>(lds, rp);
}

template <typename IT, int D, int GW, int DK>
static void launch_rd(bool delta, const RecurArgs& a, hipStream_t st) {
  const int grid = a.units * (a.hsplit > 1 ? a.hsplit : 1);
  if (delta)
    hipLaunchKernelGGL((recur_kernel<IT, D, GW, DK, true>), dim3(grid), dim3(kRecurThreads), 0, st, a);
  else
    hipLaunchKernelGGL((recur_kernel<IT, D, GW, DK, false>), dim3(grid), dim3(kRecurThreads), 0, st, a);
}

template <typename IT, int D>
static void launch_rg(int G, int dk, bool delta, const RecurArgs& a, hipStream_t st) {
  auto go = [&](auto gw) {
    constexpr int GW = decltype(gw)::value;
    switch (dk) {
      case 0: launch_rd<IT, D, GW, 0>(delta, a, st); break;
      case 1: launch_rd<IT, D, GW, 1>(delta, a, st); break;
      default: launch_rd<IT, D, GW, 2>(delta, a, st); break;
    }
  };
  switch (G) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
}

hipError_t launch_recur(int io, int D, int G, int decay_kind, int delta, const RecurArgs& a, hipStream_t st) {
  if (a.units <= 0) return hipSuccess;
  // head size 128 only: the smaller ones fit the chunk kernels
  if (D != 128) return hipErrorInvalidValue;
  switch (io) {
    case kIoBF16: launch_rg<uint16_t, 128>(G, decay_kind, delta != 0, a, st); break;
    case kIoF16: launch_rg<f16_t, 128>(G, decay_kind, delta != 0, a, st); break;
    default: launch_rg<float, 128>(G, decay_kind, delta != 0, a, st); break;
  }
  return hipGetLastError();
}

}  // namespace la

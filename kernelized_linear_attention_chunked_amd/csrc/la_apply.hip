// Non-causal readout ("[Feature] LinearAttention layer for Keras", sections
// "Mathematical definition / Non-causal" and "Masking / Non-causal"): once the
// summed state (S, Z) of a (batch, head) unit is known every query is
// independent,
//   y_i = phi(q_i)^T S / (phi(q_i)^T Z + eps),   y_i = 0 for a masked query.
//
// A streaming kernel.  A workgroup copies one unit's S into LDS as the bf16 (or
// fp32) operand S^T [dv][dk], plus 16 rows holding Z, so that the normaliser
// rides in the same MFMAs as an extra output tile.  Its 8 waves then run
// through 16-row query blocks on their own, with no barrier.  Per block a wave
// loads q as whole rows (each instruction covers full 256-byte rows), applies
// phi and parks it in its own 16-row LDS tile, reads it back in MFMA operand
// layout, runs (D/16 + 1) value tiles x D/32 MFMAs against S^T, and sends the
// results out through the same tile so that the stores are whole rows too
// (the MFMA layouts alone would touch 16 rows per instruction).  Two blocks of
// q are in flight per wave, in two register sets that alternate, so that no
// register still being loaded is ever copied.  Workgroup sg of a unit takes the
// unit's blocks sg, sg + n, sg + 2n, ... (n workgroups per unit), which spreads
// masked tails evenly; a block without a valid query stores zeros and reads no q.
#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

constexpr int kApplyBlockRows = 16;
constexpr int kApplyMaxBlocksPerWave = 16;  // liveness of a wave's blocks: one ballot
constexpr int kApplyWaves = 8;
constexpr int kApplyThreads = 64 * kApplyWaves;

// PAD: Dk != Dv (a.dk, a.dv), as in the chunk kernel: D = max(Dk, Dv) wide
// tiles, q blocks past Dk read as zeros with phi 0, S rows past Dk and columns
// past Dv zero, outputs stored Dv wide.
template <typename IT, int D, int FM, bool NORM, bool MASKED, bool PAD = false>
// 16-bit operands: two workgroups per CU (at most 128 registers); fp32 S^T
// tiles at head size 128 fit the LDS once
__global__ __launch_bounds__(kApplyThreads, (sizeof(typename Io<IT>::DT) == 2 || D < 128) ? 4 : 1) void apply_kernel(ApplyArgs a) {
  using DT = typename Io<IT>::DT;  // operand type of the I/O type IT
  using O = Op<DT>;
  constexpr int VEC = O::VEC, KB = O::KB, ESZ = O::ESZ;
  constexpr int NDT = D / 16;
  constexpr int NVT = NDT + (NORM ? 1 : 0);
  constexpr int NQ = D / KB;
  constexpr int SB_LD = D + 16 / ESZ;
  constexpr int NW = kApplyWaves;
  constexpr int CB = D / VEC;                   // 16-byte blocks per row
  constexpr int NLD = kApplyBlockRows * CB / 64;  // row-wise 16-byte loads per lane per block
  static_assert(NLD >= 1 && NLD * 64 == kApplyBlockRows * CB, "whole rows per load");
  __shared__ __align__(16) DT Sb[NVT * 16 * SB_LD];
  __shared__ __align__(16) DT Stg[NW * kApplyBlockRows * SB_LD];  // per-wave 16-row tiles

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int l = tid & 63, lr = l & 15, lg = l >> 4;
  const int nseg = a.seg_count;
  const int u = blockIdx.x / nseg, sg = blockIdx.x % nseg;
  const int T = a.T, H = a.H;
  const int DKr = PAD ? a.dk : D, DVr = PAD ? a.dv : D;  // head sizes in memory
  const int HDK = H * DKr, HDV = H * DVr;
  const int b = u / H, h = u % H;
  auto sq_at = [&](int r, int col) {
    return r * SB_LD + (((col / VEC) ^ sq_swz(r)) * VEC) + (col % VEC);
  };

  // ---- S and Z -> S^T in LDS: coalesced 16-byte loads of S rows, all issued
  // before the transposed writes; a lane takes KPL consecutive dk of four
  // consecutive dv, so its LDS words run along S^T rows
  {
    const float* sin = a.s + (int64_t)u * a.s_u;
    const float* zin = NORM ? a.z + (int64_t)u * a.z_u : nullptr;
    constexpr int KPL = 4 / ESZ;
    constexpr int NCOPY = (D / 4) * (D / KPL);
    constexpr int NIT = (NCOPY + kApplyThreads - 1) / kApplyThreads;
    auto put = [&](int off, const float (&x)[KPL]) {
      if constexpr (ESZ == 2)
        *(uint32_t*)(Sb + off) = pack_bf16x2(x[0], x[1]);
      else
        ((float*)Sb)[off] = x[0];
    };
    f32x4_t x[NIT][KPL];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + it * kApplyThreads;
      const int dv = 4 * (idx / (D / KPL)), dk = KPL * (idx % (D / KPL));
#pragma unroll
      for (int p = 0; p < KPL; ++p)
        x[it][p] = (idx < NCOPY && dk + p < DKr && dv < DVr) ? *(const f32x4_t*)(sin + (dk + p) * DVr + dv)
                                                            : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int idx = tid + it * kApplyThreads;
      if (idx >= NCOPY) break;
      const int dv = 4 * (idx / (D / KPL)), dk = KPL * (idx % (D / KPL));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y[KPL];
#pragma unroll
        for (int p = 0; p < KPL; ++p) y[p] = x[it][p][j];
        put(sq_at(dv + j, dk), y);
      }
    }
    if constexpr (NORM) {
      for (int idx = tid; idx < 16 * (D / KPL); idx += kApplyThreads) {
        const int r = idx / (D / KPL), dk = KPL * (idx % (D / KPL));
        float y[KPL];
#pragma unroll
        for (int p = 0; p < KPL; ++p) y[p] = dk + p < DKr ? zin[dk + p] : 0.f;
        put(sq_at(D + r, dk), y);
      }
    }
  }

  const IT* qb = (const IT*)a.q + (int64_t)b * T * HDK + (int64_t)h * DKr;
  IT* ob = (IT*)a.out + (int64_t)b * T * HDV + (int64_t)h * DVr;
  const uint8_t* const mb = MASKED ? a.mask + (int64_t)b * T : nullptr;
  const int nblk = (T + kApplyBlockRows - 1) / kApplyBlockRows;
  // block of the wave's i-th step (may lie past the end: then it is skipped)
  auto blk_of = [&](int i) { return sg + nseg * (w + NW * i); };
  const int nsteps = (nblk - sg - nseg * w + nseg * NW - 1) / (nseg * NW);  // blocks of this wave

  // liveness of the wave's blocks: lane l checks rows 4(l%4)..4(l%4)+3 of step l/4
  uint32_t live = 0;
  {
    const int row0 = kApplyBlockRows * blk_of(l >> 2) + 4 * (l & 3);
    bool any = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = row0 + k;
      any = any || (row < T && (!MASKED || mb[row] != 0));
    }
    const uint64_t bal = __ballot(any);
#pragma unroll
    for (int i = 0; i < kApplyMaxBlocksPerWave; ++i)
      live |= (((bal >> (4 * i)) & 0xfull) != 0 ? 1u : 0u) << i;
  }

  __syncthreads();

  // the wave's LDS tile; lane l's g-th 16-byte piece of a block (g = 64k + l)
  // is row g / CB, block g % CB of it
  DT* stg = Stg + w * kApplyBlockRows * SB_LD;
  // the two register sets of raw q (row-wise) and the mask byte of the lane's query
  u32x4_t qa[NLD], qc[NLD];
  uint32_t ka = 1u, kc = 1u;
  auto load = [&](u32x4_t (&q)[NLD], uint32_t& k, int i) {
    if (i < nsteps && ((live >> i) & 1u)) {
      const int r0 = kApplyBlockRows * blk_of(i);
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int g = 64 * n + l;
        const int row = min(r0 + g / CB, T - 1);  // rows past the end read the last
        q[n] = (!PAD || (g % CB) * VEC < DKr) ? ld16(qb + (int64_t)row * HDK + (g % CB) * VEC)
                                              : u32x4_t{0u, 0u, 0u, 0u};
      }
      if constexpr (MASKED) k = mb[min(r0 + lr, T - 1)];
    }
  };
  auto process = [&](const u32x4_t (&q)[NLD], uint32_t k, int i) {
    if (i >= nsteps) return;
    // the lane indices pass through an empty asm, so that the LDS addresses
    // derived from them are formed per block, not held across the loop
    {
      int x = tid & 63;
      asm volatile("" : "+v"(x));
      l = x;
      lr = x & 15;
      lg = x >> 4;
    }
    const int r0 = kApplyBlockRows * blk_of(i);
    if (!((live >> i) & 1u)) {
#pragma unroll
      for (int n = 0; n < NLD; ++n) {
        const int g = 64 * n + l;
        if (r0 + g / CB < T && (!PAD || (g % CB) * VEC < DVr))
          st16(ob + (int64_t)(r0 + g / CB) * HDV + (g % CB) * VEC, u32x4_t{0u, 0u, 0u, 0u});
      }
      return;
    }
    const bool ok = r0 + lr < T && (!MASKED || k != 0u);
    // phi(q), parked row-wise, read back as the B operand (column = the lane's
    // query lr, contraction = dk); one wave's LDS accesses stay in order
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int g = 64 * n + l;
      float f[VEC];
      Io<IT>::unpack(q[n], f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) f[e] = phi<FM>(f[e], a.eps);
      const u32x4_t fq = O::pack(f);
      st16(stg + sq_at(g / CB, (g % CB) * VEC), (!PAD || (g % CB) * VEC < DKr) ? fq : u32x4_t{0u, 0u, 0u, 0u});
    }
    u32x4_t qop[NQ];
#pragma unroll
    for (int m = 0; m < NQ; ++m) qop[m] = ld16(stg + sq_at(lr, KB * m + VEC * lg));
    f32x4_t nacc[NVT];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) nacc[vt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const u32x4_t av = ld16(Sb + sq_at(16 * vt + lr, KB * m + VEC * lg));
        O::mma(nacc[vt], av, qop[m]);
      }
    }
    // each query is its own MFMA column, so a masked query's values (whatever
    // its q holds) reach only its own outputs, which are selected to zero
    const float rden = NORM ? 1.f / (nacc[NVT - 1][0] + a.eps) : 1.f;
#pragma unroll
    for (int vt = 0; vt < NDT; ++vt)
      store4((IT*)(stg + sq_at(lr, 16 * vt + 4 * lg)), ok ? nacc[vt][0] * rden : 0.f,
             ok ? nacc[vt][1] * rden : 0.f, ok ? nacc[vt][2] * rden : 0.f, ok ? nacc[vt][3] * rden : 0.f);
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int g = 64 * n + l;
      const u32x4_t v = ld16(stg + sq_at(g / CB, (g % CB) * VEC));
      if (r0 + g / CB < T && (!PAD || (g % CB) * VEC < DVr)) st16(ob + (int64_t)(r0 + g / CB) * HDV + (g % CB) * VEC, v);
    }
  };

  load(qa, ka, 0);
  load(qc, kc, 1);
  for (int i = 0; i < nsteps; i += 2) {
    process(qa, ka, i);
    load(qa, ka, i + 2);
    process(qc, kc, i + 1);
    load(qc, kc, i + 3);
  }
}

template <typename IT, int D, int FM, bool NORM>
static void launch_m(const ApplyArgs& a, int grid, hipStream_t st) {
  if constexpr (D > 32) {
    if (a.dk != a.dv) {
      if (a.mask)
        hipLaunchKernelGGL((apply_kernel<IT, D, FM, NORM, true, true>), dim3(grid), dim3(kApplyThreads), 0, st, a);
      else
        hipLaunchKernelGGL((apply_kernel<IT, D, FM, NORM, false, true>), dim3(grid), dim3(kApplyThreads), 0, st, a);
      return;
    }
  }
  if (a.mask)
    hipLaunchKernelGGL((apply_kernel<IT, D, FM, NORM, true>), dim3(grid), dim3(kApplyThreads), 0, st, a);
  else
    hipLaunchKernelGGL((apply_kernel<IT, D, FM, NORM, false>), dim3(grid), dim3(kApplyThreads), 0, st, a);
}

template <typename IT, int D>
static void launch_fn(int fm, int norm, const ApplyArgs& a, int grid, hipStream_t st) {
  if (fm == kEluPlusOne) {
    if (norm) launch_m<IT, D, kEluPlusOne, true>(a, grid, st);
    else launch_m<IT, D, kEluPlusOne, false>(a, grid, st);
  } else {
    if (norm) launch_m<IT, D, kReluEps, true>(a, grid, st);
    else launch_m<IT, D, kReluEps, false>(a, grid, st);
  }
}

template <typename IT>
static void launch_d(int D, int fm, int norm, const ApplyArgs& a, int grid, hipStream_t st) {
  switch (D) {
    case 32: launch_fn<IT, 32>(fm, norm, a, grid, st); break;
    case 64: launch_fn<IT, 64>(fm, norm, a, grid, st); break;
    default: launch_fn<IT, 128>(fm, norm, a, grid, st); break;
  }
}

int apply_groups_per_unit(int64_t U, int64_t T) {
  const int64_t nblk = (T + kApplyBlockRows - 1) / kApplyBlockRows;
  // every wave takes at most kApplyMaxBlocksPerWave blocks; aim at 2 workgroups
  // per CU over 256 CUs; never more workgroups than a unit has blocks
  const int64_t per_group = (int64_t)kApplyWaves * kApplyMaxBlocksPerWave;
  int64_t n = (nblk + per_group - 1) / per_group;
  const int64_t want = (512 + U - 1) / U;
  if (n < want) n = want;
  if (n > nblk) n = nblk;
  if (n < 1) n = 1;
  return (int)n;
}

hipError_t launch_apply(int io, int D, int fm, int norm, const ApplyArgs& a, int grid,
                        hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  switch (io) {
    case kIoBF16: launch_d<uint16_t>(D, fm, norm, a, grid, st); break;
    case kIoF16: launch_d<f16_t>(D, fm, norm, a, grid, st); break;
    default: launch_d<float>(D, fm, norm, a, grid, st); break;
  }
  return hipGetLastError();
}

}  // namespace la

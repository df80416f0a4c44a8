// Chunk-parallel kernels for causal and non-causal kernelized linear attention.
//
// One templated kernel, two modes (the non-causal readout with a fixed state is
// the streaming kernel of la_apply.hip):
//   kCausal : causal prefill ("[Feature] LinearAttention layer for Keras",
//             sections "Mathematical definition / Causal", "Masking / Causal",
//             "Streaming State").  Per chunk of 64 tokens it forms
//               A^T = phiK phiQ^T (lower triangle, diagonal included),
//               N^T = V^T A^T + S_prev^T phiQ^T,
//             divides by the normaliser and stores the outputs, then adds
//             phiK^T V to the running state S (carried in registers).
//   kState  : only the state increment  sum_t phiK_t^T V_t  over a segment of
//             chunks (the partial sums of a split sequence, and the non-causal
//             reduction of "Mathematical definition / Non-causal").
// The operator page ("LinearAttention", ai.onnx v27, "Description") allows any
// chunk-parallel evaluation with the sequential result; chunking changes only
// the summation order.
//
// The normaliser rides along in the same MFMAs: V^T gets 16 extra rows of
// ones and S gets 16 extra columns holding Z, so the extra output tile of
// N^T holds  sum_j A_ij + phiQ_i . Z_prev  (the denominator before eps), and
// the extra state tile accumulates Z exactly like S.
//
// Work split inside a workgroup (one (batch, head) unit and one segment of
// chunks; 4 wavefronts, or 8 at head size 128):
//   wave w owns query rows [16qr, 16qr+16) of the chunk, qr = w % 4 (reversed
//   for w >= 4, so that the two waves of a SIMD balance; A^T tiles
//   jt <= qr), and for them the output tiles of one value half (w / 4) plus the
//   normaliser tile; and a contiguous 1/NW of the 16x16 tiles of S.
// LDS holds phiK and phiQ in natural [token][d] layout, V transposed
// [dv][token] (16-byte blocks swizzled per row) and a copy of S transposed
// [dv][dk] in the operand dtype.  The next chunk's q/k/v are loaded into
// registers while the current chunk is being computed.
#include <type_traits>

#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {

enum ChunkMode { kCausal = 0, kState = 1 };

// Wavefronts per workgroup: 8 at head sizes 64 and 128 (the state and the
// output accumulators would not fit one 4-wave workgroup's registers without
// serialising every LDS read; at 64 the halved per-wave tiles let two 8-wave
// workgroups share a CU), 4 below.
template <int D>
struct ChunkWaves {
  static constexpr int NW = D >= 64 ? 8 : 4;
};

// LDS layouts: the swizzles of la_device.hpp (vt_swz, kn_swz, sq_swz).

// The second bound is the minimum number of waves per SIMD.  At 8 waves the
// bf16 state mode, and the bf16 causal mode at head size 64, ask for 4 (two
// workgroups per CU, at most 128 registers); the causal mode at 128 and the
// fp32 kernels need more registers.
template <typename DT, int D, int MODE>
struct ChunkOccupancy {
  static constexpr int NW = ChunkWaves<D>::NW;
  static constexpr int value = NW == 8 ? ((sizeof(DT) == 2 && (MODE != kCausal || D == 64)) ? 4 : 1) : 2;
};

// MASKED: a (B,T) mask is given.  Unmasked launches carry no mask code at all.
// IT: the I/O element type (Io<IT>); DT: the operand type it is computed in.
// PAD: Dk != Dv (a.dk, a.dv): the tiles are D = max(Dk, Dv) wide; q and k
// blocks past Dk load as zeros with phi selected to 0, v blocks past Dv load as
// zeros, and outputs and states are stored in their own (dk, dv) shapes.
// Without PAD the head sizes are D and no guard is compiled in.
template <typename IT, int D, int FM, bool NORM, int MODE, bool MASKED, bool PAD = false>
__global__ __launch_bounds__(64 * ChunkWaves<D>::NW, (ChunkOccupancy<IT, D, MODE>::value))
void chunk_kernel(ChunkArgs a) {
  using DT = typename Io<IT>::DT;
  using O = Op<DT>;
  constexpr int NW = ChunkWaves<D>::NW;            // wavefronts
  constexpr int NTH = 64 * NW;                     // threads
  constexpr int NH = NW / 4;                       // value halves (waves per query block)
  constexpr int VEC = O::VEC, KB = O::KB, ESZ = O::ESZ;
  constexpr int NDT = D / 16;                      // 16-wide tiles along dk or dv
  constexpr int NVT = NDT + (NORM ? 1 : 0);        // dv tiles plus the normaliser tile
  constexpr int NDH = NDT / NH;                    // dv tiles of one value half
  constexpr int NVW = NDH + (NORM ? 1 : 0);        // a wave's output tiles (+ normaliser)
  constexpr int CB = D / VEC;                      // 16-byte blocks per row
  // tokens per loading thread (bf16 V^T writes pack token pairs: at least 2)
  constexpr int LOADERS = (kChunk * CB / NTH >= 2 || ESZ == 4) ? NTH : kChunk * CB / 2;
  constexpr int NTOK = kChunk * CB / LOADERS;
  constexpr int NQ = D / KB;                       // operand vectors per q row per lane
  constexpr int NKS = kChunk / KB;                 // vector-steps over the chunk's tokens
  // 16-bit operands: unpadded phi(K), phi(Q) and S^T rows whose 16-byte
  // blocks are XORed by a function of the row (ksw, qsw); fp32: 16 bytes of
  // padding per row and the shared swizzles of la_device.hpp
  constexpr bool SWZ = ESZ == 2;
  constexpr int PADE = SWZ ? 0 : 16 / ESZ;
  constexpr int KN_LD = D + PADE;                  // phi(K), phi(Q) rows
  constexpr int VT_LD = kChunk;                    // V^T rows (swizzled, unpadded)
  constexpr int SB_LD = D + PADE;
  constexpr bool USE_KV = true;
  constexpr bool USE_Q = MODE == kCausal;
  constexpr bool USE_SB = MODE == kCausal;
  // phi(Q) is staged through LDS (each element evaluated once, coalesced
  // loads), except for fp32 at head size 128 where it would not fit: there each
  // wave loads its own query rows straight into operand registers.
  constexpr bool QS_STAGE = !(ESZ == 4 && D >= 128);
  // 16-bit operands keep phi(K) transposed as well, [dk][token] like V^T, so
  // that each state-update operand is one 16-byte read; the row-major phi(K)
  // remains for the causal A^T tiles (and for the fp32 update; the causal
  // kernel at smaller head sizes keeps its occupancy without it)
  constexpr bool KT = USE_KV && ESZ == 2 && (D >= 128 || MODE == kState);
  constexpr bool KN_ROWS = USE_KV && (MODE == kCausal || !KT);
  constexpr int KN_BYTES = KN_ROWS ? kChunk * KN_LD * ESZ : 0;
  constexpr int QS_BYTES = (USE_Q && QS_STAGE) ? kChunk * KN_LD * ESZ : 0;
  constexpr int VT_BYTES = USE_KV ? NVT * 16 * VT_LD * ESZ : 0;
  constexpr int SB_BYTES = USE_SB ? NVT * 16 * SB_LD * ESZ : 0;
  // fp16 inputs: V is staged as hi + lo bf16 tiles (every fp16 value is the
  // exact sum of two bf16 values), and each product with V takes one more MFMA
  // with the lo tile, so that V reaches the products unrounded
  constexpr bool VLO = !std::is_same_v<IT, DT>;
  // lane indices re-derived per chunk where that removes spills (head size 64;
  // fp32 and fp16 inputs at head size 128, the bf16 state pass): elsewhere it
  // measured slower
  constexpr bool REFRESH = D == 64 || (D >= 128 && (ESZ == 4 || VLO || MODE == kState));
  constexpr int VL_BYTES = (USE_KV && VLO) ? NDT * 16 * VT_LD * ESZ : 0;
  constexpr int KT_BYTES = KT ? D * VT_LD * ESZ : 0;
  constexpr int NS = NDT * NVT;                    // 16x16 tiles of the (extended) state
  constexpr int TPW = (NS + NW - 1) / NW;          // state tiles per wave
  static_assert(NTOK >= 1 && NQ >= 1 && NDH * NH == NDT, "unsupported head size");
  static_assert(ESZ == 4 || NTOK % 2 == 0, "bf16 V^T writes pack token pairs");
  static_assert(SB_LD == KN_LD, "phi(Q) and S^T share one row layout");

  __shared__ __align__(16) unsigned char smem[KN_BYTES + QS_BYTES + VT_BYTES + SB_BYTES + VL_BYTES + KT_BYTES + 16];
  DT* Kn = (DT*)smem;
  DT* Qs = (DT*)(smem + KN_BYTES);
  DT* Vt = (DT*)(smem + KN_BYTES + QS_BYTES);
  DT* Sb = (DT*)(smem + KN_BYTES + QS_BYTES + VT_BYTES);
  DT* Vl = (DT*)(smem + KN_BYTES + QS_BYTES + VT_BYTES + SB_BYTES);
  DT* Kt = (DT*)(smem + KN_BYTES + QS_BYTES + VT_BYTES + SB_BYTES + VL_BYTES);  // phi(K)^T (KT)

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // query rows [16qr, 16qr+16) of the chunk and value half hv (dv tiles
  // [hv*NDH, (hv+1)*NDH), plus the normaliser tile).  Waves w and w + 4 share a
  // SIMD; giving them row blocks qr and 3 - qr evens out the causal work.
  const int qr = (w & 4) ? 3 - (w & 3) : (w & 3);
  const int hv = w >> 2;
  int l = tid & 63, lr = l & 15, lg = l >> 4;
  auto refresh = [&]() {
    if constexpr (REFRESH) {
      l = opaque_lane(tid);
      lr = l & 15;
      lg = l >> 4;
    }
  };
  const int bid = blockIdx.x;
  const int u = bid / a.seg_count;
  const int s = a.seg_first + bid % a.seg_count;
  const int H = a.H, T = a.T;
  const int b = u / H, h = u % H;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const int cstep = a.chunk_step > 1 ? a.chunk_step : 1;
  const int c0 = cstep > 1 ? s : s * a.seg_chunks;
  const int c1 = cstep > 1 ? nchunks : min(c0 + a.seg_chunks, nchunks);
  const int DKr = PAD ? a.dk : D, DVr = PAD ? a.dv : D;  // head sizes in memory
  const int HDK = H * DKr, HDV = H * DVr;                 // token strides of q/k and v/out
  const IT* qb = (const IT*)a.q + (int64_t)b * T * HDK + (int64_t)h * DKr;
  const IT* kb = (const IT*)a.k + (int64_t)b * T * HDK + (int64_t)h * DKr;
  const IT* vb = (const IT*)a.v + (int64_t)b * T * HDV + (int64_t)h * DVr;
  IT* ob = (IT*)a.out + (int64_t)b * T * HDV + (int64_t)h * DVr;
  const uint8_t* const mb = MASKED ? a.mask + (int64_t)b * T : nullptr;
  const float eps = a.eps;
  // global dv tile of the wave's i-th output tile
  auto vtile = [&](int i) { return (NORM && i == NDH) ? NDT : hv * NDH + i; };
  // element offset of 16-byte block `blk` of V^T row r
  auto vt_at = [&](int r, int blk) { return r * VT_LD + ((blk ^ vt_swz(r)) * VEC); };
  // element offset of element `col` of phi(K) row t: 16-byte blocks swizzled by
  // row bits 3 and 4 so that the permuted-row operand reads (rows t and t+8 in
  // one pass) and the column-wise reads of the state update (rows 8 apart)
  // spread over the banks
  auto kn_at = [&](int t, int col) {
    const int sw = SWZ ? ksw<CB>(t) : (kn_swz(t) & (CB - 1));
    return t * KN_LD + ((((col / VEC) ^ sw) & (CB - 1)) * VEC) + (col % VEC);
  };
  // element offset of element `col` of row r of phi(Q) or S^T
  auto sq_at = [&](int r, int col) {
    const int sw = SWZ ? qsw<CB>(r) : sq_swz(r);
    return r * SB_LD + ((((col / VEC) ^ sw) & (CB - 1)) * VEC) + (col % VEC);
  };

  // ---- running state.  With FUSE, wave (qr, hv) owns state rows
  // [R*qr, R*qr+R) across its own value tiles (the normaliser column belongs to
  // half 0), so the V^T operands it loads for the intra-chunk product serve the
  // state update too; otherwise wave w owns tiles w*TPW .. w*TPW+TPW-1.
  constexpr bool FUSE = NDT % 4 == 0;
  constexpr int R = FUSE ? NDT / 4 : 1;
  constexpr int NST = FUSE ? R * NVW : TPW;
  auto stile = [&](int k, int& rt, int& ct) -> bool {
    if constexpr (FUSE) {
      const int j = k / NVW, i = k % NVW;
      rt = R * qr + j;
      ct = vtile(i);
      return hv == 0 || i < NDH;
    } else {
      const int tau = w * TPW + k;
      rt = tau / NVT;
      ct = tau % NVT;
      return tau < NS;
    }
  };
  f32x4_t sacc[NST];
#pragma unroll
  for (int k = 0; k < NST; ++k) sacc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (MODE == kCausal) {
    // (head size 128 keeps the prefix pass: its registers have no room for the
    // batched slot loads)
    constexpr bool FOLD = D <= 64;
    // the segment's start state: its prefixed slot, or (fold) the initial
    // state plus the unprefixed slots 1 .. s in slot order, every slot's loads
    // issued before the adds
    const bool fold = FOLD && a.fold != 0;
    const float* sin = fold ? (a.s_init ? a.s_init + u * a.s_init_u : nullptr)
                            : (a.s_in ? a.s_in + u * a.s_in_u + s * a.s_in_s : nullptr);
    const float* zin = fold ? (a.z_init ? a.z_init + u * a.z_init_u : nullptr)
                            : (a.z_in ? a.z_in + u * a.z_in_u + s * a.z_in_s : nullptr);
    const float* sl = (fold && a.s_in) ? a.s_in + u * a.s_in_u : nullptr;
    const float* zl = (fold && a.z_in) ? a.z_in + u * a.z_in_u : nullptr;
    const int R = sl ? s : 0;
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      int rt, ct;
      if (stile(k, rt, ct)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dk = 16 * rt + 4 * lg + q;
          const bool sv = ct < NDT && dk < DKr && 16 * ct + lr < DVr, zv = ct >= NDT && dk < DKr;
          const int64_t o = ct < NDT ? (int64_t)dk * DVr + 16 * ct + lr : dk;
          const float* b = ct < NDT ? sin : zin;
          const float* lb = ct < NDT ? sl : zl;
          const int64_t ls = ct < NDT ? a.s_in_s : a.z_in_s;
          constexpr int NF = FOLD ? kChunkFold - 1 : 1;
          float y[NF];
#pragma unroll
          for (int r = 1; r <= NF; ++r) y[r - 1] = (r <= R && lb && (sv || zv)) ? lb[r * ls + o] : 0.f;
          float val = ((sv || zv) && b) ? b[o] : 0.f;
#pragma unroll
          for (int r = 1; r <= NF; ++r)
            if (r <= R) val += y[r - 1];
          sacc[k][q] = val;
        }
      }
    }
  }

  // S (and Z in the extra rows) -> LDS, transposed [dv][dk], operand dtype.
  auto write_sb = [&]() {
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      int rt, ct;
      if (stile(k, rt, ct)) {
        DT* p = Sb + sq_at(16 * ct + lr, 16 * rt + 4 * lg);
        if constexpr (ESZ == 2) {
          u32x2_t v2;
          v2[0] = pack_bf16x2(sacc[k][0], sacc[k][1]);
          v2[1] = pack_bf16x2(sacc[k][2], sacc[k][3]);
          *(u32x2_t*)p = v2;
        } else {
          *(f32x4_t*)p = sacc[k];
        }
      }
    }
  };
  if constexpr (MODE == kCausal) write_sb();
  if constexpr (USE_KV && NORM) {
    // rows D..D+15 of V^T are ones: they turn A V into the row sums of A
    for (int idx = tid; idx < 16 * VT_LD; idx += NTH) {
      if constexpr (ESZ == 2)
        ((uint16_t*)Vt)[D * VT_LD + idx] = 0x3f80;  // bf16 1.0
      else
        ((float*)Vt)[D * VT_LD + idx] = 1.f;
    }
  }

  // ---- prefetch registers: thread (cb, tg) loads the 16-byte block cb of
  // NTOK consecutive tokens tg*NTOK + n, for q, k and v alike (full rows per
  // 16 threads: coalesced).  Where the loaders are half the workgroup and q is
  // staged (QSPLIT), the other half loads and stages q (into pk), so that
  // phi(q) and phi(k) are evaluated by different waves.
  constexpr bool QSPLIT = USE_Q && QS_STAGE && 2 * LOADERS == NTH;
  const bool qload = QSPLIT && tid >= LOADERS;  // (wave-uniform: LOADERS is a multiple of 64)
  const int lt = qload ? tid - LOADERS : tid;
  const int cb = lt % CB, tg = lt / CB;
  const bool loader = LOADERS == NTH || tid < LOADERS || QSPLIT;
  // the loader's 16-byte block lies inside the q/k rows (kin) and v rows (vin)
  const bool kin = !PAD || cb * VEC < DKr, vin = !PAD || cb * VEC < DVr;
  const u32x4_t zero4 = u32x4_t{0u, 0u, 0u, 0u};
  u32x4_t pk[USE_KV ? NTOK : 1], pv[USE_KV ? NTOK : 1];
  u32x4_t pq[USE_Q ? (QS_STAGE ? (QSPLIT ? 1 : NTOK) : NQ) : 1];
  u32x4_t qreg[(USE_Q && !QS_STAGE) ? NQ : 1];
  uint32_t valid = 0;   // bit n: token tg*NTOK + n exists and is not masked
  bool qrow_ok = false; // (unstaged q) this lane's own query row exists and is not masked
  // the prefetched chunk holds at least one valid token (plive) / every token
  // exists and is valid (pfull); the same in every wave (each ballots the
  // chunk's 64 mask bytes), so the branches on them are uniform
  bool plive = true, pfull = true;
  static_assert(kChunk == 64, "one mask byte per lane");
  // mask byte of token l of the chunk prefetched next, loaded one chunk ahead
  // so that the ballot does not wait on it
  auto load_mask = [&](int c) -> uint32_t {
    const int t = c * kChunk + l;
    return (c < c1 && t < T) ? (uint32_t)mb[t] : 0u;
  };
  uint32_t mnext = (mb && c0 < c1) ? load_mask(c0) : 0u;
  auto prefetch = [&](int c) {
    const int tb = c * kChunk;
    valid = 0;
    pfull = tb + kChunk <= T;
    if (mb) {
      const uint64_t bal = __ballot(mnext != 0u);
      plive = bal != 0;
      pfull = pfull && bal == ~0ull;
      mnext = load_mask(c + cstep);
      if (!plive) return;  // fully masked chunk: nothing to load
    }
    if constexpr (USE_Q && !QS_STAGE) {
      const int tok = tb + 16 * qr + lr;
      qrow_ok = tok < T && (mb ? (mb[tok] != 0) : true);
#pragma unroll
      for (int m = 0; m < NQ; ++m)
        pq[m] = (tok < T && (!PAD || KB * m + VEC * lg < DKr)) ? ld16(qb + (int64_t)tok * HDK + KB * m + VEC * lg)
                                                            : zero4;
    }
    if (!loader) return;
    if constexpr (QSPLIT) {
      if (qload) {
        // the q half: the same tokens' q blocks, into pk
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
          const int tok = tb + tg * NTOK + n;
          const bool in = pfull || tok < T;
          pk[n] = (kin && in) ? ld16(qb + (int64_t)tok * HDK + cb * VEC) : zero4;
          const uint32_t ok = pfull ? 1u : (in ? (mb ? (mb[tok] != 0) : 1u) : 0u);
          valid |= ok << n;
        }
        return;
      }
    }
    if (pfull) {
      // whole chunk, every token valid: no per-token guards
      valid = (1u << NTOK) - 1u;
#pragma unroll
      for (int n = 0; n < NTOK; ++n) {
        const int64_t tok = tb + tg * NTOK + n;
        const int64_t offk = tok * HDK + cb * VEC, offv = tok * HDV + cb * VEC;
        if constexpr (USE_KV) {
          pk[n] = kin ? ld16(kb + offk) : zero4;
          pv[n] = vin ? ld16(vb + offv) : zero4;
        }
        if constexpr (USE_Q && QS_STAGE && !QSPLIT) pq[n] = kin ? ld16(qb + offk) : zero4;
      }
      return;
    }
#pragma unroll
    for (int n = 0; n < NTOK; ++n) {
      const int tok = tb + tg * NTOK + n;
      if (tok < T) {
        const int64_t offk = (int64_t)tok * HDK + cb * VEC, offv = (int64_t)tok * HDV + cb * VEC;
        if constexpr (USE_KV) {
          pk[n] = kin ? ld16(kb + offk) : zero4;
          pv[n] = vin ? ld16(vb + offv) : zero4;
        }
        if constexpr (USE_Q && QS_STAGE && !QSPLIT) pq[n] = kin ? ld16(qb + offk) : zero4;
        const uint32_t ok = mb ? (mb[tok] != 0) : 1u;
        valid |= ok << n;
      } else {
        if constexpr (USE_KV) {
          pk[n] = u32x4_t{0u, 0u, 0u, 0u};
          pv[n] = u32x4_t{0u, 0u, 0u, 0u};
        }
        if constexpr (USE_Q && QS_STAGE && !QSPLIT) pq[n] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };

  // phi of one 16-byte block, then zero if the token is invalid (selected on
  // the packed words: a masked token must not reach anything, whatever its values)
  auto phi_vec = [&](const u32x4_t& raw, bool ok, auto full) {
    float f[VEC];
    Io<IT>::unpack(raw, f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) f[e] = phi<FM>(f[e], eps);
    u32x4_t r = O::pack(f);
    if constexpr (!decltype(full)::value) {
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = ok ? r[e] : 0u;
    }
    return r;
  };

  // V -> V^T [dv][token] (swizzled) at `base`: element e of every loaded vector
  // goes to V^T row cb*VEC + e; the thread's NTOK consecutive tokens sit side by
  // side (a thread's tokens may span several 16-byte blocks, which the swizzle
  // does not keep adjacent: each group is addressed by itself)
  auto write_vt = [&](DT* base, const u32x4_t (&src)[NTOK]) {
    const int t0 = tg * NTOK;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int r = cb * VEC + e;
      if constexpr (ESZ == 2) {
#pragma unroll
        for (int n = 0; n < NTOK; n += 2) {
          const uint32_t w0 = src[n][e >> 1], w1 = src[n + 1][e >> 1];
          // low halves of both words for even e, high halves for odd e
          *(uint32_t*)(base + vt_at(r, (t0 + n) / VEC) + (t0 + n) % VEC) =
              (e & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u) : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
        }
      } else {
        float fv[NTOK];
#pragma unroll
        for (int n = 0; n < NTOK; ++n) fv[n] = __uint_as_float(src[n][e]);
        DT* p = base + vt_at(r, t0 / VEC) + (t0 % VEC);
        if constexpr (NTOK == 1) {
          *(float*)p = fv[0];
        } else if constexpr (NTOK == 2) {
          *(float2*)p = make_float2(fv[0], fv[1]);
        } else {
#pragma unroll
          for (int n = 0; n < NTOK; n += 4)
            *(f32x4_t*)(base + vt_at(r, (t0 + n) / VEC)) = f32x4_t{fv[n], fv[n + 1], fv[n + 2], fv[n + 3]};
        }
      }
    }
  };

  // ---- stage: phi(K), phi(Q) -> [token][d] in LDS, V -> V^T [dv][token] (swizzled).
  // `full` (a std::bool_constant) marks a whole unmasked chunk: no validity selects.
  auto stage = [&](auto full) {
    constexpr bool FULL = decltype(full)::value;
    if constexpr (USE_Q && !QS_STAGE) {
#pragma unroll
      for (int m = 0; m < NQ; ++m)
        qreg[m] = (!PAD || KB * m + VEC * lg < DKr) ? phi_vec(pq[m], qrow_ok, full) : zero4;
    }
    if (!loader) return;
    if constexpr (QSPLIT) {
      if (qload) {
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
          const bool ok = FULL || ((valid >> n) & 1u);
          st16(Qs + sq_at(tg * NTOK + n, cb * VEC), kin ? phi_vec(pk[n], ok, full) : zero4);
        }
        return;
      }
    }
    u32x4_t pkt[KT ? NTOK : 1];
#pragma unroll
    for (int n = 0; n < NTOK; ++n) {
      const bool ok = FULL || ((valid >> n) & 1u);
      const int t = tg * NTOK + n;
      if constexpr (USE_KV) {
        const u32x4_t fk = kin ? phi_vec(pk[n], ok, full) : zero4;
        if constexpr (KN_ROWS) st16(Kn + kn_at(t, cb * VEC), fk);
        if constexpr (KT) pkt[n] = fk;
        if (!ok) pv[n] = u32x4_t{0u, 0u, 0u, 0u};
      }
      if constexpr (USE_Q && QS_STAGE && !QSPLIT) st16(Qs + sq_at(t, cb * VEC), kin ? phi_vec(pq[n], ok, full) : zero4);
    }
    if constexpr (USE_KV) {
      if constexpr (VLO) {
        u32x4_t pl[NTOK];
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
          float f[VEC];
          Io<IT>::unpack(pv[n], f);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t hw = pack_bf16x2(f[2 * i], f[2 * i + 1]);
            pv[n][i] = hw;
            pl[n][i] = pack_bf16x2(f[2 * i] - __uint_as_float(hw << 16),
                                   f[2 * i + 1] - __uint_as_float(hw & 0xffff0000u));
          }
        }
        write_vt(Vl, pl);
      }
      write_vt(Vt, pv);
      if constexpr (KT) write_vt(Kt, pkt);
    }
  };

  // ---- per-chunk compute
  // phiK^T operand of the state update for state row rt, token block m (lane
  // group lg carries tokens KB*m + VEC*lg + e), read column-wise from phi(K)
  auto load_kop = [&](u32x4_t& dst, int rt, int m) {
    const int t0 = KB * m + VEC * lg, col = 16 * rt + lr;
    if constexpr (KT) {
      dst = ld16(Kt + vt_at(col, (KB / VEC) * m + lg));  // one row of phi(K)^T
    } else if constexpr (ESZ == 2) {
      const uint16_t* k16 = (const uint16_t*)Kn;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dst[e] = (uint32_t)k16[kn_at(t0 + 2 * e, col)] | ((uint32_t)k16[kn_at(t0 + 2 * e + 1, col)] << 16);
    } else {
      const float* k32 = (const float*)Kn;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = __float_as_uint(k32[kn_at(t0 + e, col)]);
    }
  };
  // V^T operand (16-byte block `blk` of row 16*ct + lr)
  auto vt_op = [&](int ct, int blk) { return ld16(Vt + vt_at(16 * ct + lr, blk)); };
  // its lo part (fp16 inputs; value tiles only, the normaliser's ones are exact)
  auto vl_op = [&](int ct, int blk) { return ld16(Vl + vt_at(16 * ct + lr, blk)); };

  auto compute = [&](int c, bool live, bool full) {
    refresh();
    if (!live) {
      // fully masked chunk: state unchanged, outputs zero
      if constexpr (USE_Q) {
        const int tok = c * kChunk + 16 * qr + lr;
        if (tok < T) {
          IT* orow = ob + (int64_t)tok * HDV + 4 * lg;
#pragma unroll
          for (int i = 0; i < NDH; ++i)
            if (!PAD || 16 * (hv * NDH + i) < DVr) store4(orow + 16 * (hv * NDH + i), 0.f, 0.f, 0.f, 0.f);
        }
      }
      return;
    }
    if constexpr (USE_Q) {
      u32x4_t qop[NQ];
#pragma unroll
      for (int m = 0; m < NQ; ++m)
        qop[m] = QS_STAGE ? ld16(Qs + sq_at(16 * qr + lr, KB * m + VEC * lg)) : qreg[m];
      f32x4_t nacc[NVW];
#pragma unroll
      for (int i = 0; i < NVW; ++i) nacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // N^T += S^T phiQ^T (state before this chunk): contraction over dk.
#pragma unroll
      for (int m = 0; m < NQ; ++m) {
        u32x4_t av[NVW];
#pragma unroll
        for (int i = 0; i < NVW; ++i) av[i] = ld16(Sb + sq_at(16 * vtile(i) + lr, KB * m + VEC * lg));
#pragma unroll
        for (int i = 0; i < NVW; ++i) O::mma(nacc[i], av[i], qop[m]);
      }
      // A^T, per key block p (= token block of the update): bf16 pairs of tiles
      // over keys [32p, 32p+32), row r of tile (p, odd) being key
      // 32p + 8(r/4) + 4odd + r%4 so that lane group lg holds keys
      // 32p + 8lg + (0..7), one 16-byte V^T read per value tile; fp32 single
      // tiles over keys [16p, 16p+16).  bf16 A is kept as hi + lo: phi >= 0
      // gives it a large common part, and one rounding would dominate the error.
      constexpr int NP = NKS;
      u32x4_t bh[NP], bl[NP];
      f32x4_t at32[ESZ == 4 ? NP : 1];
      auto need = [&](int p) { return (ESZ == 2) ? (32 * p <= 16 * qr + 15) : (p <= qr); };
      if constexpr (MODE == kCausal) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          if (!need(p)) continue;
          f32x4_t at[2];
#pragma unroll
          for (int odd = 0; odd < (ESZ == 2 ? 2 : 1); ++odd) {
            const int krow = (ESZ == 2) ? 32 * p + 8 * (lr >> 2) + 4 * odd + (lr & 3) : 16 * p + lr;
            u32x4_t kv[NQ];
#pragma unroll
            for (int m = 0; m < NQ; ++m) kv[m] = ld16(Kn + kn_at(krow, KB * m + VEC * lg));
            at[odd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NQ; ++m) O::mma(at[odd], kv[m], qop[m]);
            // causal: key <= query, only where the key block reaches past the
            // block's first query (below it every key is earlier)
            if ((ESZ == 2 ? 32 * p + 31 : 16 * p + 15) > 16 * qr) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int key = (ESZ == 2) ? 32 * p + 8 * lg + 4 * odd + q : 16 * p + 4 * lg + q;
                at[odd][q] = (key <= 16 * qr + lr) ? at[odd][q] : 0.f;
              }
            }
          }
          if constexpr (ESZ == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x0 = at[e >> 1][2 * (e & 1)], x1 = at[e >> 1][2 * (e & 1) + 1];
              const uint32_t hw = pack_bf16x2(x0, x1);
              bh[p][e] = hw;
              bl[p][e] = pack_bf16x2(x0 - __uint_as_float(hw << 16), x1 - __uint_as_float(hw & 0xffff0000u));
            }
          } else {
            at32[p] = at[0];
          }
        }
      }
      // state-update operands of the wave's rows
      u32x4_t kop[FUSE ? R : 1][NKS];
      if constexpr (FUSE) {
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
          for (int m = 0; m < NKS; ++m) load_kop(kop[j][m], R * qr + j, m);
      }
      // per key/token block: V^T operands -> intra-chunk product and state update
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const bool intra = (MODE == kCausal) && need(p);
        if (!intra && !FUSE) continue;
        u32x4_t av[NVW];
#pragma unroll
        for (int i = 0; i < NVW; ++i) av[i] = vt_op(vtile(i), (KB / VEC) * p + lg);
        u32x4_t avl[VLO ? NDH : 1];
        if constexpr (VLO) {
#pragma unroll
          for (int i = 0; i < NDH; ++i) avl[i] = vl_op(vtile(i), (KB / VEC) * p + lg);
        }
        if (intra) {
#pragma unroll
          for (int i = 0; i < NVW; ++i) {
            if constexpr (ESZ == 2) {
              O::mma(nacc[i], av[i], bh[p]);
              O::mma(nacc[i], av[i], bl[p]);
              if constexpr (VLO) {
                if (i < NDH) O::mma(nacc[i], avl[i], bh[p]);
              }
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                nacc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av[i][q]), at32[p][q],
                                                               nacc[i], 0, 0, 0);
            }
          }
        }
        if constexpr (FUSE) {
#pragma unroll
          for (int j = 0; j < R; ++j)
#pragma unroll
            for (int i = 0; i < NVW; ++i)
              if (hv == 0 || i < NDH) O::mma(sacc[j * NVW + i], kop[j][p], av[i]);
          if constexpr (VLO) {
#pragma unroll
            for (int j = 0; j < R; ++j)
#pragma unroll
              for (int i = 0; i < NDH; ++i) O::mma(sacc[j * NVW + i], kop[j][p], avl[i]);
          }
        }
      }
      // epilogue: lane holds query 16qr + lr, value dims 16*vtile(i) + 4lg + (0..3)
      const int tok = c * kChunk + 16 * qr + lr;
      if (tok < T) {
        const bool ok = (full || !mb) ? true : (mb[tok] != 0);
        float rden = 1.f;
        if constexpr (NORM) rden = ok ? __builtin_amdgcn_rcpf(nacc[NDH][0] + eps) : 0.f;  // (v_rcp_f32: 1 ulp)
        else rden = ok ? 1.f : 0.f;
        IT* orow = ob + (int64_t)tok * HDV + 4 * lg;
#pragma unroll
        for (int i = 0; i < NDH; ++i)
          if (!PAD || 16 * (hv * NDH + i) < DVr)
            store4(orow + 16 * (hv * NDH + i), nacc[i][0] * rden, nacc[i][1] * rden,
                   nacc[i][2] * rden, nacc[i][3] * rden);
      }
    }
    if constexpr (USE_KV && !(FUSE && USE_Q)) {
      // S += phiK^T V on its own (state-only mode, or no fused assignment)
      u32x4_t kop[NKS];
      int cur_rt = -1;
#pragma unroll
      for (int k = 0; k < NST; ++k) {
        int rt, ct;
        if (stile(k, rt, ct)) {
          if (rt != cur_rt) {
            cur_rt = rt;
#pragma unroll
            for (int m = 0; m < NKS; ++m) load_kop(kop[m], rt, m);
          }
          u32x4_t bv[NKS];
#pragma unroll
          for (int m = 0; m < NKS; ++m) bv[m] = vt_op(ct, (KB / VEC) * m + lg);
#pragma unroll
          for (int m = 0; m < NKS; ++m) O::mma(sacc[k], kop[m], bv[m]);
          if constexpr (VLO) {
            if (ct < NDT) {
#pragma unroll
              for (int m = 0; m < NKS; ++m) O::mma(sacc[k], kop[m], vl_op(ct, (KB / VEC) * m + lg));
            }
          }
        }
      }
    }
  };

  if (c0 < c1) prefetch(c0);
  for (int c = c0; c < c1; c += cstep) {
    const bool live = MASKED ? plive : true;
    const bool full = pfull;
    if (live) {
      if (full)
        stage(std::true_type{});
      else
        stage(std::false_type{});
      __syncthreads();
    }
    if (c + cstep < c1) prefetch(c + cstep);
    // a dead chunk touches no LDS, so it needs neither barrier: the next
    // chunk's stage cannot overwrite anything a slower wave still reads
    compute(c, live, full);
    if (live) {
      __syncthreads();
      if constexpr (MODE == kCausal) write_sb();
    }
  }

  // ---- state out
  float* sout = nullptr;
  float* zout = nullptr;
  if constexpr (MODE == kCausal) {
    if (s == a.nseg_total - 1) {
      sout = a.s_out ? a.s_out + u * a.s_out_u : nullptr;
      zout = a.z_out ? a.z_out + u * a.z_out_u : nullptr;
    }
  } else if constexpr (MODE == kState) {
    sout = a.s_out + u * a.s_out_u + (s + a.out_slot_off) * a.s_out_s;
    zout = a.z_out ? a.z_out + u * a.z_out_u + (s + a.out_slot_off) * a.z_out_s : nullptr;
  }
  {
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      int rt, ct;
      if (stile(k, rt, ct)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dk = 16 * rt + 4 * lg + q;
          if (ct < NDT) {
            if (sout && dk < DKr && 16 * ct + lr < DVr) sout[dk * DVr + 16 * ct + lr] = sacc[k][q];
          } else {
            if (zout && lr == 0 && dk < DKr) zout[dk] = sacc[k][q];
          }
        }
      }
    }
  }
}

// Exclusive prefix over segment partial states, in place.  Slot s of unit u
// holds the increment of segment s-1 on entry (slot 0 is ignored) and the
// state before segment s on exit; slot 0 receives the caller's initial state
// (or zeros).  One thread per four consecutive state elements (D is a multiple
// of 4, so a group never straddles the S and Z parts), sequential over
// segments.  Every load of a batch of 16 slots is issued before the batch's
// stores, so a unit takes one memory round trip per batch rather than one per
// segment; slots past the last are clamped to it and their values unused.
constexpr int kSegBatch = 16;

__global__ __launch_bounds__(kThreads) void seg_prefix_kernel(float* ws_s, float* ws_z,
                                                              const float* s_in, const float* z_in,
                                                              int U, int nseg, int dk, int dv, int norm) {
  const int SE = dk * dv;  // floats of S per slot (a multiple of 4, like dk)
  const int64_t per4 = ((int64_t)SE + (norm ? dk : 0)) / 4;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)U * per4) return;
  const int u = (int)(idx / per4);
  const int e = 4 * (int)(idx % per4);
  f32x4_t* base;
  int64_t stride;  // in 4-element groups
  const f32x4_t* init;
  if (e < SE) {
    base = (f32x4_t*)(ws_s + (int64_t)u * nseg * SE + e);
    stride = SE / 4;
    init = s_in ? (const f32x4_t*)(s_in + (int64_t)u * SE + e) : nullptr;
  } else {
    const int ez = e - SE;
    base = (f32x4_t*)(ws_z + (int64_t)u * nseg * dk + ez);
    stride = dk / 4;
    init = z_in ? (const f32x4_t*)(z_in + (int64_t)u * dk + ez) : nullptr;
  }
  f32x4_t acc = init ? *init : f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t x[kSegBatch];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j) x[j] = base[min(s0 + j, nseg - 1) * stride];
  };
  if (nseg > 1) load_batch(1);
  base[0] = acc;
  for (int s0 = 1; s0 < nseg; s0 += kSegBatch) {
    if (s0 > 1) load_batch(s0);
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j) {
      if (s0 + j < nseg) {
        acc += x[j];
        base[(s0 + j) * stride] = acc;
      }
    }
  }
}

// Sum of all segment partials of a unit, in fixed segment order, into slot 0
// (four consecutive elements per thread, a batch of slots in flight at a time).
__global__ __launch_bounds__(kThreads) void seg_sum_kernel(float* ws_s, float* ws_z, int U,
                                                           int nseg, int dk, int dv, int norm) {
  const int SE = dk * dv;
  const int64_t per4 = ((int64_t)SE + (norm ? dk : 0)) / 4;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)U * per4) return;
  const int u = (int)(idx / per4);
  const int e = 4 * (int)(idx % per4);
  f32x4_t* base;
  int64_t stride;
  if (e < SE) {
    base = (f32x4_t*)(ws_s + (int64_t)u * nseg * SE + e);
    stride = SE / 4;
  } else {
    base = (f32x4_t*)(ws_z + (int64_t)u * nseg * dk + (e - SE));
    stride = dk / 4;
  }
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nseg; s0 += kSegBatch) {
    f32x4_t x[kSegBatch];
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j) x[j] = base[min(s0 + j, nseg - 1) * stride];
#pragma unroll
    for (int j = 0; j < kSegBatch; ++j)
      if (s0 + j < nseg) acc += x[j];
  }
  base[0] = acc;
}

// ---------------------------------------------------------------------------
// host-side launchers

template <typename IT, int D, int FM, bool NORM, int MODE>
static hipError_t launch_one(const ChunkArgs& a, int grid, hipStream_t st) {
  const dim3 blk(64 * ChunkWaves<D>::NW);
  if constexpr (D > 32) {
    if (a.dk != a.dv) {
      if (a.mask)
        hipLaunchKernelGGL((chunk_kernel<IT, D, FM, NORM, MODE, true, true>), dim3(grid), blk, 0, st, a);
      else
        hipLaunchKernelGGL((chunk_kernel<IT, D, FM, NORM, MODE, false, true>), dim3(grid), blk, 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.mask)
    hipLaunchKernelGGL((chunk_kernel<IT, D, FM, NORM, MODE, true>), dim3(grid), blk, 0, st, a);
  else
    hipLaunchKernelGGL((chunk_kernel<IT, D, FM, NORM, MODE, false>), dim3(grid), blk, 0, st, a);
  return hipGetLastError();
}

template <typename IT, int D, int FM, bool NORM>
static hipError_t launch_mode(int mode, const ChunkArgs& a, int grid, hipStream_t st) {
  return mode == kCausal ? launch_one<IT, D, FM, NORM, kCausal>(a, grid, st)
                         : launch_one<IT, D, FM, NORM, kState>(a, grid, st);
}

template <typename IT, int D>
static hipError_t launch_d(int mode, int fm, int norm, const ChunkArgs& a, int grid, hipStream_t st) {
  if (fm == kEluPlusOne)
    return norm ? launch_mode<IT, D, kEluPlusOne, true>(mode, a, grid, st)
                : launch_mode<IT, D, kEluPlusOne, false>(mode, a, grid, st);
  return norm ? launch_mode<IT, D, kReluEps, true>(mode, a, grid, st)
              : launch_mode<IT, D, kReluEps, false>(mode, a, grid, st);
}

template <typename IT>
static hipError_t launch_dt(int mode, int D, int fm, int norm, const ChunkArgs& a, int grid,
                            hipStream_t st) {
  switch (D) {
    case 32: return launch_d<IT, 32>(mode, fm, norm, a, grid, st);
    case 64: return launch_d<IT, 64>(mode, fm, norm, a, grid, st);
    default: return launch_d<IT, 128>(mode, fm, norm, a, grid, st);
  }
}

hipError_t launch_chunk(int mode, int io, int D, int fm, int norm, const ChunkArgs& a, int grid,
                        hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  switch (io) {
    case kIoBF16: return launch_dt<uint16_t>(mode, D, fm, norm, a, grid, st);
    case kIoF16: return launch_dt<f16_t>(mode, D, fm, norm, a, grid, st);
    default: return launch_dt<float>(mode, D, fm, norm, a, grid, st);
  }
}

hipError_t launch_seg_prefix(float* ws_s, float* ws_z, const float* s_in, const float* z_in, int U,
                             int nseg, int dk, int dv, int norm, hipStream_t st) {
  const int64_t n = (int64_t)U * ((int64_t)dk * dv + (norm ? dk : 0)) / 4;
  const int grid = (int)((n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(seg_prefix_kernel, dim3(grid), dim3(kThreads), 0, st, ws_s, ws_z, s_in, z_in,
                     U, nseg, dk, dv, norm);
  return hipGetLastError();
}

hipError_t launch_seg_sum(float* ws_s, float* ws_z, int U, int nseg, int dk, int dv, int norm,
                          hipStream_t st) {
  const int64_t n = (int64_t)U * ((int64_t)dk * dv + (norm ? dk : 0)) / 4;
  const int grid = (int)((n + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(seg_sum_kernel, dim3(grid), dim3(kThreads), 0, st, ws_s, ws_z, U, nseg, dk, dv, norm);
  return hipGetLastError();
}

}  // namespace la

// gdr_bwd.hip -- backward kernels of the chunked gated delta rule on gfx950.
//
// The backward of the FlashQLA pages ("FlashQLA Documentation", backward
// pass: dq, dk, dv, db, dg, dh0 from q, k, v, g, beta, A, do, dht).  The
// forward's chunk states are not an input, so they are recomputed.
//
//   B1  scan (forward, state mode)   chunk-start states S_c       -> h  (ws)
//   B2  dh_scan (reverse)            with dSn the gradient of a chunk's end
//       state:   dDelta = diag(e^{gL-gamma}) K dSn + scale P^T dO
//                dS     = e^{gL} dSn + Q^T (scale diag(e^gamma) dO)
//                         - K^T diag(beta e^gamma) A^T dDelta
//       stores dSn per chunk (-> dh, ws) and dh0; long sequences are split
//       along T with the transposed segment transitions (same augmented-
//       state construction as the forward).
//   B3-5 grad_kernel, one workgroup per (chunk, value head), from S and dSn:
//       R = diag(beta) V - diag(beta e^gamma) K S, Delta = A R,
//       dDelta (as above), dR = A^T dDelta, dM = strict_lower(-dR Delta^T)
//       (the gradient of A = (I + M)^-1 is -A^T dA A^T with dA = dDelta R^T,
//       and A^T dDelta R^T A^T = dR Delta^T), dP = scale lower_incl(dO Delta^T),
//       dq = scale diag(e^gamma) dO S^T + (dP o Gamma) K
//       dk = (dP o Gamma)^T Q + diag(e^{gL-gamma}) Delta dSn^T
//            - diag(beta e^gamma) dR S^T + (dM o beta Gamma) K + (..)^T K
//       dv = diag(beta) dR, dbeta and dgamma by fixed-order row reductions,
//       dg = reverse chunk-local cumsum of dgamma (times the gate's slope when
//       g is a gate input, with per-chunk shares of the gate parameters'
//       gradients, summed per head by gate_param_grad_kernel).
//   B6  with GVA the gradient kernel runs twice: value heads 0 .. G-2 of each
//       group leave fp32 dq, dk rows in workspace slots, head G-1 adds them in
//       head order to its own and stores dq, dk once.
#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_scan.h"

#include <algorithm>
#include <type_traits>
#include <cstring>

namespace gdr {

// ---------------------------------------------------------------------------
// B2: reverse recurrence of the state gradient
// ---------------------------------------------------------------------------
struct DhArgs {
  const void* q;
  const void* k;
  const void* dO;
  const void* beta;
  const float* gcum;
  const void* A;
  const float* dht;    // [N, Hv, K, V] (svf aware), nullable
  void* dh;            // [NC, Hv] packed (packed_off), in_dtype: gradient of each chunk's end state
  float* dh0;          // nullable (svf aware)
  const float* seg_start;  // [units, P, K, V]: gradient entering each segment's end
  float* seg_out;          // [units, P, K, 2V]: augmented pass-1 results
  const int32_t* cu;
  const int32_t* offs;
  const int32_t* order;  // packed input: sequences by chunk count, longest first (block_pos)
  int N, T, Hq, Hv, nc_dense;
  int P, nvs;
  float scale;
  int svf;
  int qk_norm;    // q, k rows scaled to unit length before use
  // (qk_norm) the rows were normalised beforehand: q and k hold the unit
  // rows, and these their 1 / |x| per (token, q head) row; else null
  const float* qinv;
  const float* kinv;
  int beta_mode;  // bit 0 sigmoid of a beta logit, bit 1 twice beta
  int v_only;     // pass 1 runs the value columns only: the transitions are
                  // the forward's, kept (ScanArgs::trans)
  // Pipelined output pass (sliced != 0): one launch runs segment slice_p of
  // every (sequence, head), the segments walked one launch after another
  // from the last; a segment starts from the gradient the launch before
  // left in seg_start and leaves its own start gradient in seg_next for
  // segment slice_p - 1 (both [units, P, K, V] fp32, one buffer).
  int sliced, slice_p, sl_c0, sl_c1;  // sliced: the slice's chunks [sl_c0, sl_c1)
  float* seg_next;
  // Gradient workgroups in the same launch (bwd_dyn_kernel, loader-wave form
  // only): per (unit, column block) the number of chunks, counted from the
  // sequence's end, whose state gradient is stored; the stores and the count
  // are coherent across the XCDs (sc1).  Null otherwise.
  unsigned* flags;
};

template <typename T, int VB, int MODE>
__device__ __forceinline__ void dh_body(const DhArgs& a, int b, int nb) {
  typedef typename VT<T>::x8 x8;
  constexpr int CW = 64 * VB;
  constexpr int LD = 136;
  constexpr int LDV = CW + 8;
  constexpr int LDA = 72;
  constexpr bool OUT = (MODE == MODE_OUT);
  __shared__ __align__(16) T Qs[64 * LD];
  __shared__ __align__(16) T Ks[64 * LD];
  __shared__ __align__(16) T Ds[64 * LDV];
  __shared__ __align__(16) T As[64 * LDA];
  __shared__ __align__(16) float gam[64], eg[64], bex[64], dl[64];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;
  const BlockPos bp = block_pos(a.order, b, nb, a.P * a.nvs, a.Hv);
  const int vs = bp.sub % a.nvs;
  const int p = bp.sub / a.nvs, unit = bp.unit;
  const int n = unit / a.Hv, h = unit % a.Hv;
  const int G = a.Hv / a.Hq, hq = h / G;
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int nch = (int)((s.end - s.start + kChunk - 1) / kChunk);
  const SegRange sr = seg_range(nch, a.P, p);
  const int cb0 = vs * CW + ((MODE == MODE_AUG && a.v_only) ? kDim : 0);
  const bool isT = (MODE == MODE_AUG) && cb0 < kDim;
  if (MODE == MODE_AUG) {
    if (p == 0 || p > sr.p_last) return;       // segment 0 needs no transition
    if (p == sr.p_last && isT) return;         // the last segment starts from dht
  } else {
    if (sr.c0 >= sr.c1 && !(nch == 0 && p == 0)) return;
  }
  const int vcol0 = (MODE == MODE_AUG) ? (isT ? 0 : cb0 - kDim) : cb0;
  const int64_t choff = a.cu ? (int64_t)a.offs[n] : (int64_t)n * a.nc_dense;
  const int64_t KV = (int64_t)kDim * kDim;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* dO = reinterpret_cast<const T*>(a.dO);
  const T* Ag = reinterpret_cast<const T*>(a.A);
  const T* beta = reinterpret_cast<const T*>(a.beta);
  const int cw0 = 16 * VB * w;

  // gradient entering the segment's end: dht (last segment) or the chained
  // value; every load is issued before the first is used (null reads zeros)
  f32x4 Gs[8][VB];
  if (MODE == MODE_AUG && isT) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Gs[kb][vb][e] = (16 * kb + 4 * grp + e == cb0 + cw0 + 16 * vb + col) ? 1.f : 0.f;
  } else {
    // the value columns of an inner segment's transition start from zero
    // (their end state is b_seg); the gradient entering it comes from pass 2
    const float* src = (p == sr.p_last) ? (a.dht ? a.dht + unit * KV : nullptr)
                       : (MODE == MODE_AUG) ? nullptr
                                            : a.seg_start + ((int64_t)unit * a.P + p) * KV;
    const bool vf = (p == sr.p_last) && a.svf;
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(src, src ? KV * (int64_t)sizeof(float) : 0);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 16 * kb + 4 * grp + e, vc = vcol0 + cw0 + 16 * vb + col;
          Gs[kb][vb][e] = buf_load_f32(srs, (vf ? vc * kDim + key : key * kDim + vc) * (int)sizeof(float));
        }
  }

  TileRegs<128, 256> rq, rk;
  TileRegs<CW, 256> rd;
  TileRegs<64, 256> ra;
  float r_g = 0.f, r_gl = 0.f;
  T r_b = from_f<T>(0.f);
  bool r_ok = false;  // the row is inside the chunk
  auto prefetch = [&](int c) {
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int Cc = (int)min((int64_t)kChunk, s.end - t0);
    if (!isT) tile_load<T, 128, 256>(rq, q + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc);
    tile_load<T, 128, 256>(rk, k + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc);
    if (!isT) tile_load<T, CW, 256>(rd, dO + (t0 * a.Hv + h) * kDim + vcol0, (int64_t)a.Hv * kDim, Cc);
    tile_load<T, 64, 256>(ra, Ag + (t0 * a.Hv + h) * kChunk, (int64_t)a.Hv * kChunk, Cc);
    if (tid < 64) {
      r_g = a.gcum[(t0 + min(tid, Cc - 1)) * a.Hv + h];
      r_gl = a.gcum[(t0 + Cc - 1) * a.Hv + h];
      r_b = (tid < Cc) ? beta[(t0 + tid) * a.Hv + h] : from_f<T>(0.f);
      r_ok = tid < Cc;
    }
  };

  // the initial state has arrived before the loop (else the loop-entry merge
  // makes the first use of Gs wait for the prefetch as well)
  __builtin_amdgcn_s_waitcnt(0);
  if (sr.c0 < sr.c1) prefetch(sr.c1 - 1);
  for (int c = sr.c1 - 1; c >= sr.c0; --c) {
    if (a.qk_norm) {
      if (!isT) l2norm_rows<T, 256>(rq, nullptr);
      l2norm_rows<T, 256>(rk, nullptr);
    }
    __syncthreads();
    if (!isT) tile_store<T, 128, 256>(Qs, LD, rq);
    tile_store<T, 128, 256>(Ks, LD, rk);
    if (!isT) tile_store<T, CW, 256>(Ds, LDV, rd);
    tile_store<T, 64, 256>(As, LDA, ra);
    if (tid < 64) {
      const float e = __expf(r_g);
      gam[tid] = r_g;
      eg[tid] = a.scale * e;
      bex[tid] = (r_ok ? beta_used(to_f(r_b), a.beta_mode) : 0.f) * e;
      dl[tid] = __expf(r_gl - r_g);
    }
    __syncthreads();
    const float eL = __expf(gam[63]);

    // gradient of this chunk's end state out, packed (packed_off)
    if (OUT) {
      const __amdgpu_buffer_rsrc_t hrs =
          buf_rsrc(reinterpret_cast<T*>(a.dh) + ((choff + c) * a.Hv + h) * KV, KV * (int64_t)sizeof(T));
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          const x8 f = pack_split<T>(Gs[2 * kb2][vb], Gs[2 * kb2 + 1][vb]);
          buf_store16(hrs, packed_off((cb0 + cw0) / 16 + vb, kb2, l) * (int)sizeof(T),
                      __builtin_bit_cast(uint4, f));
        }
    }

    // One pass over the key dimension forms K dSn and the lower tiles of
    // P = Q K^T (tile (rb, ib), ib <= rb: rows r = 16 rb + 4 grp + e, column
    // i = 16 ib + col) from the same K fragments.
    x8 Gb[4][VB];
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) Gb[kb2][vb] = pack_split<T>(Gs[2 * kb2][vb], Gs[2 * kb2 + 1][vb]);
    f32x4 dd[4][VB], pt[10];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) dd[tb][vb] = zero4();
#pragma unroll
    for (int x = 0; x < 10; ++x) pt[x] = zero4();
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) {
      x8 fk[4], fq[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) fk[tb] = frag_row_split(Ks + 16 * tb * LD + 32 * kb2, LD);
      if (!isT) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) fq[tb] = frag_row_split(Qs + 16 * tb * LD + 32 * kb2, LD);
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) dd[tb][vb] = mfma16(fk[tb], Gb[kb2][vb], dd[tb][vb]);
      if (!isT) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int ib = 0; ib <= rb; ++ib) pt[tri_idx(ib, rb)] = mfma16(fq[rb], fk[ib], pt[tri_idx(ib, rb)]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c - 1 >= sr.c0) prefetch(c - 1);

    // dDelta = diag(e^{gL-gamma}) K dSn + scale P^T dO.  Two stacked D tiles
    // of P (rows r) form the A operand of P^T with k = r.
    if (!isT) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const f32x4 gr = *reinterpret_cast<const f32x4*>(gam + 16 * rb + 4 * grp);
#pragma unroll
        for (int ib = 0; ib <= rb; ++ib) {
          const float gi = gam[16 * ib + col];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // masked entries take exp(-inf) = 0 (unconditional exponential)
            const bool keep = (ib < rb) || (col <= 4 * grp + e);
            pt[tri_idx(ib, rb)][e] *= __expf(keep ? gr[e] - gi : -INFINITY);
          }
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      x8 pa[2];
#pragma unroll
      for (int kt = tb / 2; kt < 2; ++kt)
        pa[kt] = pack_split<T>((2 * kt >= tb) ? pt[tri_idx(tb, 2 * kt < 4 ? 2 * kt : 3)] : zero4(),
                               pt[tri_idx(tb, 2 * kt + 1)]);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        f32x4 acc = zero4();
        if (!isT) {
#pragma unroll
          for (int kt = tb / 2; kt < 2; ++kt)
            acc = mfma16(pa[kt], frag_tr_split(Ds + 32 * kt * LDV + cw0 + 16 * vb, LDV), acc);
        }
        const f32x4 dlr = *reinterpret_cast<const f32x4*>(dl + 16 * tb + 4 * grp);
#pragma unroll
        for (int e = 0; e < 4; ++e) dd[tb][vb][e] = dlr[e] * dd[tb][vb][e] + a.scale * acc[e];
      }
    }
    // Z = -diag(beta e^gamma) A^T dDelta
    f32x4 zz[4][VB];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kt = tb / 2; kt < 2; ++kt)
          acc = mfma16(frag_tr_split(As + 32 * kt * LDA + 16 * tb, LDA),
                       pack_split<T>(dd[2 * kt][vb], dd[2 * kt + 1][vb]), acc);
        const f32x4 bx = *reinterpret_cast<const f32x4*>(bex + 16 * tb + 4 * grp);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= -bx[e];
        zz[tb][vb] = acc;
      }
    // dS = e^{gL} dSn + K^T Z + Q^T (scale diag(e^gamma) dO)
    x8 Zb[2][VB], Ob[2][VB];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        Zb[kt][vb] = pack_split<T>(zz[2 * kt][vb], zz[2 * kt + 1][vb]);
        if (!isT) {
          x8 f = frag_tr_split(Ds + 32 * kt * LDV + cw0 + 16 * vb, LDV);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int r = 32 * kt + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
            f[e] = from_f<T>(to_f(f[e]) * eg[r]);
          }
          Ob[kt][vb] = f;
        }
      }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      x8 fk[2], fq[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        fk[kt] = frag_tr_split(Ks + 32 * kt * LD + 16 * kb, LD);
        if (!isT) fq[kt] = frag_tr_split(Qs + 32 * kt * LD + 16 * kb, LD);
      }
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        f32x4 acc = Gs[kb][vb] * eL;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          acc = mfma16(fk[kt], Zb[kt][vb], acc);
          if (!isT) acc = mfma16(fq[kt], Ob[kt][vb], acc);
        }
        Gs[kb][vb] = acc;
      }
    }
  }

  if (MODE == MODE_AUG) {
    float* so = a.seg_out + ((int64_t)unit * a.P + p) * (2 * KV);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          so[(16 * kb + 4 * grp + e) * (2 * kDim) + cb0 + cw0 + 16 * vb + col] = Gs[kb][vb][e];
  } else if (p == 0 && a.dh0) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 16 * kb + 4 * grp + e, vc = vcol0 + cw0 + 16 * vb + col;
          a.dh0[unit * KV + (a.svf ? vc * kDim + key : key * kDim + vc)] = Gs[kb][vb][e];
        }
  }
}

// B2 output pass (one 64-column block, 8 waves).  Waves 0-3 run the chain;
// waves 4-7 issue every chunk load and tile store.  The q / k tiles and the
// per-row values of two chunks are kept (slot = chunk & 1).  In the
// iteration of chunk c, before the middle barrier, the helpers store chunk
// c's dO and A tiles (dO also scaled by scale e^gamma, the operand of Q^T),
// chunk c-1's q / k slot and chunk c+1's dSn, while the chain waves form
// K dSn and, each a quarter of its tiles, P of chunk c; after it the chain
// finishes chunk c in rounds of independent products and the helpers issue
// the loads of the next chunks.
// LDS of one B2 output-pass workgroup (dh_lh_body), a struct so that a
// launch can share its LDS with another pass's workgroups.
template <typename T>
struct DhLhLds {
  static constexpr int CW = 64, LD = 136, LDV = CW + 8, LDA = 72;
  alignas(16) T Qs[2][64 * LD];
  alignas(16) T Ks[2][64 * LD];
  alignas(16) T Ds[64 * LDV];
  alignas(16) T Es[64 * LDV];  // scale diag(e^gamma) dO
  alignas(16) T As[64 * LDA];
  alignas(16) T Ps[64 * LDA];
  alignas(16) float gam[2][64];
  alignas(16) float eg[2][64];
  alignas(16) float bex[2][64];
  alignas(16) float dl[2][64];
  // dSn of the chain's chunk as bf16 operand registers ([column block][k
  // block][lane]), stored by the helpers in the next iteration
  alignas(16) typename VT<T>::x8 Hx[4][4][64];
};

template <typename T, int OPT>
__device__ __forceinline__ void dh_lh_body(const DhArgs& a, int b, int nb, DhLhLds<T>& L) {
  typedef typename VT<T>::x8 x8;
  constexpr int CW = DhLhLds<T>::CW;
  constexpr int LD = DhLhLds<T>::LD;
  constexpr int LDV = DhLhLds<T>::LDV;
  constexpr int LDA = DhLhLds<T>::LDA;
  auto& Qs = L.Qs;
  auto& Ks = L.Ks;
  auto& Ds = L.Ds;
  auto& Es = L.Es;
  auto& As = L.As;
  auto& Ps = L.Ps;
  auto& gam = L.gam;
  auto& eg = L.eg;
  auto& bex = L.bex;
  auto& dl = L.dl;
  auto& Hx = L.Hx;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;
  const bool helper = w >= 4;
  const int otid = tid - 256;  // index among the helper threads
  // a pipelined slice runs one segment of every unit
  const BlockPos bp = block_pos(a.order, b, nb, a.sliced ? a.nvs : a.P * a.nvs, a.Hv);
  const int vs = bp.sub % a.nvs;
  const int p = a.sliced ? a.slice_p : bp.sub / a.nvs, unit = bp.unit;
  const int n = unit / a.Hv, h = unit % a.Hv;
  const int G = a.Hv / a.Hq, hq = h / G;
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int nch = (int)((s.end - s.start + kChunk - 1) / kChunk);
  SegRange sr = seg_range(nch, a.P, p);
  if (a.sliced) {  // a dense batch: every sequence has the same slices
    sr.c0 = a.sl_c0;
    sr.c1 = a.sl_c1;
    sr.p_last = a.P - 1;
  }
  if (sr.c0 >= sr.c1 && !(nch == 0 && p == 0)) return;
  const int cb0 = vs * CW;
  const int64_t choff = a.cu ? (int64_t)a.offs[n] : (int64_t)n * a.nc_dense;
  const int64_t KV = (int64_t)kDim * kDim;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* dO = reinterpret_cast<const T*>(a.dO);
  const T* Ag = reinterpret_cast<const T*>(a.A);
  const T* beta = reinterpret_cast<const T*>(a.beta);
  const int cw0 = 16 * (w & 3);

  // gradient entering the segment's end: dht (last segment) or the value
  // chained by pass 2; every load is issued before the first is used (null
  // reads zeros)
  f32x4 Gs[8];
  {
    const float* src = (p == sr.p_last) ? (a.dht ? a.dht + unit * KV : nullptr)
                                        : a.seg_start + ((int64_t)unit * a.P + p) * KV;
    const bool vf = (p == sr.p_last) && a.svf;
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(src, src ? KV * (int64_t)sizeof(float) : 0);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 16 * kb + 4 * grp + e, vc = cb0 + cw0 + col;
        Gs[kb][e] = buf_load_f32(srs, (vf ? vc * kDim + key : key * kDim + vc) * (int)sizeof(float));
      }
  }

  TileRegs<128, 256> rq, rk;
  TileRegs<CW, 256> rd;
  TileRegs<64, 256> ra;
  float r_g = 0.f, r_gl = 0.f;
  T r_b = from_f<T>(0.f);
  bool r_ok = false;  // the row is inside the chunk
  auto chunk_rows = [&](int c) { return (int)min((int64_t)kChunk, s.end - s.start - (int64_t)kChunk * c); };
  // q, k tiles and per-row values of chunk c
  auto load_qk = [&](int c) {
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int Cc = chunk_rows(c);
    tile_load<T, 128, 256>(rq, q + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc, otid);
    tile_load<T, 128, 256>(rk, k + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc, otid);
    if (otid < 64) {
      r_g = a.gcum[(t0 + min(otid, Cc - 1)) * a.Hv + h];
      r_gl = a.gcum[(t0 + Cc - 1) * a.Hv + h];
      r_b = (otid < Cc) ? beta[(t0 + otid) * a.Hv + h] : from_f<T>(0.f);
      r_ok = otid < Cc;
    }
  };
  auto store_qk = [&](int c) {
    const int b = c & 1;
    if (OPT & 1) {
      l2norm_rows<T, 256>(rq, nullptr, otid);
      l2norm_rows<T, 256>(rk, nullptr, otid);
    }
    tile_store<T, 128, 256>(Qs[b], LD, rq, otid);
    tile_store<T, 128, 256>(Ks[b], LD, rk, otid);
    if (otid < 64) {
      const float e = __expf(r_g);
      gam[b][otid] = r_g;
      eg[b][otid] = a.scale * e;
      bex[b][otid] = ((OPT & 2) ? (r_ok ? beta_used(to_f(r_b), a.beta_mode) : 0.f) : to_f(r_b)) * e;
      dl[b][otid] = __expf(r_gl - r_g);
    }
  };
  // dO and A tiles of chunk c
  auto load_da = [&](int c) {
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int Cc = chunk_rows(c);
    tile_load<T, CW, 256>(rd, dO + (t0 * a.Hv + h) * kDim + cb0, (int64_t)a.Hv * kDim, Cc, otid);
    tile_load<T, 64, 256>(ra, Ag + (t0 * a.Hv + h) * kChunk, (int64_t)a.Hv * kChunk, Cc, otid);
  };

  // gradient of chunk cc's end state out, packed (packed_off), from the
  // operand copy the chain left in Hx; non-temporal, as this pass never
  // reads it back
  auto store_dh = [&](int cc) {
    const int wq = w & 3;
    const __amdgpu_buffer_rsrc_t hrs =
        buf_rsrc(reinterpret_cast<T*>(a.dh) + ((choff + cc) * a.Hv + h) * KV, KV * (int64_t)sizeof(T));
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2)
      buf_store16_nt(hrs, packed_off(cb0 / 16 + wq, kb2, l) * (int)sizeof(T),
                  __builtin_bit_cast(uint4, Hx[wq][kb2][l]));
  };

  // the initial gradient has arrived before the loop (else the loop-entry
  // merge makes its first use wait for the helpers' loads as well)
  __builtin_amdgcn_s_waitcnt(0);
  // the two tiles above the diagonal that P^T's products read stay zero
  p_zero_tiles<T>(Ps, LDA);
  if (helper && sr.c0 < sr.c1) {
    const int cf = sr.c1 - 1;
    load_da(cf);
    load_qk(cf);
    store_qk(cf);
    if (cf - 1 >= sr.c0) load_qk(cf - 1);
  }
  // this chain wave's P tiles (as in p_tiles): 3, 3, 2, 2 per wave, (row
  // block, column block) 4 bits each
  constexpr uint64_t pcode = 0x0000ull | (0x8ull << 4) | (0xFull << 8) |
                             ((0x4ull | (0x5ull << 4) | (0xCull << 8)) << 16) |
                             ((0x9ull | (0xAull << 4)) << 32) |
                             ((0xDull | (0xEull << 4)) << 48);
  const int wu = __builtin_amdgcn_readfirstlane(w & 3);
  for (int c = sr.c1 - 1; c >= sr.c0; --c) {
    const int b = c & 1;
    __syncthreads();  // chunk c's slot is ready; every wave is done with chunk c+1
    f32x4 dd[4];
    if (helper) {
      tile_store<T, CW, 256>(Ds, LDV, rd, otid);
      tile_store<T, 64, 256>(As, LDA, ra, otid);
      // the dO tile scaled by scale e^gamma of its row (chunk c's per-row
      // values were stored one iteration earlier), the B operand of Q^T
#pragma unroll
      for (int i = 0; i < TileRegs<CW, 256>::N; ++i) {
        constexpr int PR = TileRegs<CW, 256>::PER_ROW;
        const int x = otid + i * 256, r = x / PR, c8 = (x % PR) * 8;
        const float f = eg[b][r];
        x8 v = __builtin_bit_cast(x8, rd.r[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = from_f<T>(to_f(v[e]) * f);
        *reinterpret_cast<x8*>(Es + r * LDV + c8) = v;
      }
      if (c - 1 >= sr.c0) store_qk(c - 1);
      // last: a later wait on this wave's vector memory counter would also
      // wait for these stores
      if (c + 1 < sr.c1) store_dh(c + 1);
    } else {
      // K dSn and this wave's tiles of P = lower_incl(Q K^T o Gamma) of
      // chunk c (published by the middle barrier), in four rounds over the
      // key dimension; every fragment of a round is read before it
      // multiplies.  P contracts over the keys, so the split k order of the
      // K dSn fragments serves it too.
      x8 Gb[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) Gb[kb2] = pack_split<T>(Gs[2 * kb2], Gs[2 * kb2 + 1]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) dd[tb] = zero4();
      const int nt = wu < 2 ? 3 : 2;
      int prb[3], pcb[3];
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int x = (int)((pcode >> (16 * wu + 4 * t)) & 15);
        prb[t] = x >> 2;
        pcb[t] = x & 3;
      }
      f32x4 pacc[3] = {zero4(), zero4(), zero4()};
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        x8 fk[4], fq[3];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) fk[tb] = frag_row_split(Ks[b] + 16 * tb * LD + 32 * kb2, LD);
#pragma unroll
        for (int t = 0; t < 3; ++t)
          if (t < nt) fq[t] = frag_row_split(Qs[b] + 16 * prb[t] * LD + 32 * kb2, LD);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) dd[tb] = mfma16(fk[tb], Gb[kb2], dd[tb]);
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          if (t < nt) {
            // the K fragment of column block pcb[t] (wave-uniform) is one of fk
            const int cb = pcb[t];
            const x8 kf = cb == 0 ? fk[0] : cb == 1 ? fk[1] : cb == 2 ? fk[2] : fk[3];
            pacc[t] = mfma16(fq[t], kf, pacc[t]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        if (t < nt) {
          const int rb = prb[t], cb = pcb[t];
          const f32x4 gr = *reinterpret_cast<const f32x4*>(gam[b] + 16 * rb + 4 * grp);
          const float gi = gam[b][16 * cb + col];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * grp + e, i = 16 * cb + col;
            // masked entries take exp(-inf) = 0 (an unconditional exponential)
            const float pv = pacc[t][e] * __expf((rb != cb || i <= r) ? gr[e] - gi : -INFINITY);
            Ps[r * LDA + i] = from_f<T>(pv);
          }
        }
      }
    }
    __syncthreads();  // P, dO and A of chunk c and chunk c-1's slot are in LDS; Hx is free
    if (helper) {
      if (c - 1 >= sr.c0) {
        load_da(c - 1);
        if (c - 2 >= sr.c0) load_qk(c - 2);
      }
      continue;
    }
    // chunk c's dSn for the helpers (packed again rather than kept live
    // across the barrier)
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) Hx[w][kb2][l] = pack_split<T>(Gs[2 * kb2], Gs[2 * kb2 + 1]);
    const float eL = __expf(gam[b][63]);

    // The products below run in rounds of independent accumulators whose
    // LDS fragments are issued before the round multiplies; the scheduling
    // fences keep the compiler from sinking every read to its product, which
    // would put one LDS latency per MFMA on the chain.
    // Fragment (tb, kt) of P^T or A^T (k = rows 32 kt ..) for kt >= tb / 2.
    auto tk = [](int tb, int kt) { return tb < 2 ? 2 * tb + kt : 2 + tb; };
    x8 fdo[2], fp[6], fa[6], fr[8];
    f32x4 dlv[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) fdo[kt] = frag_tr_split(Ds + 32 * kt * LDV + cw0, LDV);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int kt = tb / 2; kt < 2; ++kt)
        fp[tk(tb, kt)] = frag_tr_split(Ps + 32 * kt * LDA + 16 * tb, LDA);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) dlv[tb] = *reinterpret_cast<const f32x4*>(dl[b] + 16 * tb + 4 * grp);
    __builtin_amdgcn_sched_barrier(0);
    // dDelta = diag(e^{gL-gamma}) K dSn + scale P^T dO
    f32x4 pd[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) pd[tb] = zero4();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        if (kt >= tb / 2) pd[tb] = mfma16(fp[tk(tb, kt)], fdo[kt], pd[tb]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int kt = tb / 2; kt < 2; ++kt)
        fa[tk(tb, kt)] = frag_tr_split(As + 32 * kt * LDA + 16 * tb, LDA);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) dd[tb][e] = dlv[tb][e] * dd[tb][e] + a.scale * pd[tb][e];
    const x8 Db[2] = {pack_split<T>(dd[0], dd[1]), pack_split<T>(dd[2], dd[3])};
    __builtin_amdgcn_sched_barrier(0);
    x8 Ob[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) Ob[kt] = frag_tr_split(Es + 32 * kt * LDV + cw0, LDV);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) fr[kb] = frag_tr_split(Qs[b] + 16 * kb, LD);
    __builtin_amdgcn_sched_barrier(0);
    // Z = -diag(beta e^gamma) A^T dDelta
    f32x4 zz[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) zz[tb] = zero4();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        if (kt >= tb / 2) zz[tb] = mfma16(fa[tk(tb, kt)], Db[kt], zz[tb]);
    // dS = e^{gL} dSn + Q^T (scale diag(e^gamma) dO) + K^T Z
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) Gs[kb] = mfma16(fr[kb], Ob[0], Gs[kb] * eL);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) fr[kb] = frag_tr_split(Qs[b] + 32 * LD + 16 * kb, LD);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const f32x4 bx = *reinterpret_cast<const f32x4*>(bex[b] + 16 * tb + 4 * grp);
#pragma unroll
      for (int e = 0; e < 4; ++e) zz[tb][e] *= -bx[e];
    }
    const x8 Zb[2] = {pack_split<T>(zz[0], zz[1]), pack_split<T>(zz[2], zz[3])};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) Gs[kb] = mfma16(fr[kb], Ob[1], Gs[kb]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) fr[kb] = frag_tr_split(Ks[b] + 32 * kt * LD + 16 * kb, LD);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) Gs[kb] = mfma16(fr[kb], Zb[kt], Gs[kb]);
    }
  }

  // the dSn of the last chunk walked (c0)
  __syncthreads();
  if (helper) {
    if (sr.c0 < sr.c1) store_dh(sr.c0);
    return;
  }
  if (p == 0 && a.dh0) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 16 * kb + 4 * grp + e, vc = cb0 + cw0 + col;
        a.dh0[unit * KV + (a.svf ? vc * kDim + key : key * kDim + vc)] = Gs[kb][e];
      }
  } else if (a.sliced && p > 0) {
    // the gradient entering the previous segment's end, for the next launch
    float* dst = a.seg_next + ((int64_t)unit * a.P + p - 1) * KV;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dst[(16 * kb + 4 * grp + e) * kDim + cb0 + cw0 + col] = Gs[kb][e];
  }
}

// B2 output pass with a loader wave (one 64-column block, 8 waves): the
// form used unless q / k are normalised in the kernel.  Waves 0-3 run the
// chain as in dh_lh_body; wave 4 copies the tiles from HBM into LDS with
// LDS-direct loads (no registers, no tile stores): in the iteration of chunk
// c, chunk c-1's dO and A tiles and per-row values before the middle
// barrier, and chunk c-2's q and k tiles after it, so that each copy has a
// chunk's time or more to land.  Its waits name how many of its
// newest copies may still be in flight (the vector memory counter retires
// loads in order).  Waves 5-7 form the P tiles of the chunk while the chain
// forms K dSn and e^{gL} dSn + Q^T (scale diag(e^gamma) dO), which need no P;
// wave 5 first stores the state gradients from the chain's operand copies.  The tiles are swizzled (sw_off),
// q / k three-deep (slot c % 3), the rest two-deep (slot c & 1); the chain
// scales the dO fragments of Q^T (scale diag(e^gamma) dO) itself.
// dSn of the chain's chunk as bf16 operand registers ([column block][k
// block][lane]), stored by wave 5 in the next iteration (64-column form only)
template <typename T, bool HAS>
struct DhLdHx {
  alignas(16) typename VT<T>::x8 Hx[4][4][64];
};
template <typename T>
struct DhLdHx<T, false> {};

// NB: 16-column blocks per chain wave (the workgroup's columns: 64 NB)
template <typename T, int NB = 1>
struct DhLdLds : DhLdHx<T, NB == 1> {
  static constexpr int CW = 64 * NB, LDA = 72;
  alignas(16) T Qs[3][64 * 128];
  alignas(16) T Ks[3][64 * 128];
  alignas(16) T Ds[2][64 * CW];
  alignas(16) T As[2][64 * 64];
  alignas(16) T Ps[64 * LDA];
  alignas(16) float gam[2][64];
  alignas(16) float eg[2][64];
  alignas(16) float bex[2][64];
  alignas(16) float dl[2][64];
};

// INST only separates the instantiations of the kernels that run the body
// (each then has one caller: with two, the compiler's inlining order changes
// and the kernel spilled 11 more registers, 7 us at B=2 T=4096 H=32)
template <typename T, int OPT, int NB = 1, int INST = 0>
__device__ __forceinline__ void dh_ld_body(const DhArgs& a, int b, int nb, DhLdLds<T, NB>& L) {
  typedef typename VT<T>::x8 x8;
  static_assert((OPT & 1) == 0, "q / k normalisation runs in dh_lh_body");
  static_assert(NB == 1 || NB == 2, "one or two column blocks per chain wave");
  // OPT bit 2: pass 1 of a split backward given the forward's transitions.
  // Segments 1 .. p_last walk their chunks from zero (the last from dht) and
  // leave the gradient reaching their start in the value half of seg_out
  // ([units, P, K, 2V]); no state gradient is stored.
  constexpr bool P1 = (OPT & 4) != 0;
  static_assert(!P1 || NB == 2, "pass 1 runs the 128-column form");
  constexpr int CW = DhLdLds<T, NB>::CW;
  constexpr int LDA = DhLdLds<T, NB>::LDA;
  auto& Qs = L.Qs;
  auto& Ks = L.Ks;
  auto& Ds = L.Ds;
  auto& As = L.As;
  auto& Ps = L.Ps;
  auto& gam = L.gam;
  auto& eg = L.eg;
  auto& bex = L.bex;
  auto& dl = L.dl;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;
  // a pipelined slice runs one segment of every unit
  const BlockPos bp = block_pos(a.order, b, nb, a.sliced ? a.nvs : a.P * a.nvs, a.Hv);
  const int vs = bp.sub % a.nvs;
  const int p = a.sliced ? a.slice_p : bp.sub / a.nvs, unit = bp.unit;
  const int n = unit / a.Hv, h = unit % a.Hv;
  const int G = a.Hv / a.Hq, hq = h / G;
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int nch = (int)((s.end - s.start + kChunk - 1) / kChunk);
  SegRange sr = seg_range(nch, a.P, p);
  if (a.sliced) {  // a dense batch: every sequence has the same slices
    sr.c0 = a.sl_c0;
    sr.c1 = a.sl_c1;
    sr.p_last = a.P - 1;
  }
  if (P1 && (p == 0 || p > sr.p_last)) return;  // segment 0 needs no pass 1
  if (sr.c0 >= sr.c1 && !(nch == 0 && p == 0)) return;
  const int cb0 = vs * CW;
  const int64_t choff = a.cu ? (int64_t)a.offs[n] : (int64_t)n * a.nc_dense;
  const int64_t KV = (int64_t)kDim * kDim;
  // chain wave w's 16-column blocks: w, w + 4 (columns cb0 + cw(j) ..)
  auto cw = [&](int j) { return 16 * ((w & 3) + 4 * j); };
  // The lane index the chain's fragment addresses derive from: in the
  // 128-column form an opaque copy per phase, so that the compiler computes
  // the swizzled addresses where they are used instead of hoisting every one
  // of them out of the loop (they would hold the registers the wider chain
  // needs and spill)
  auto fresh_lane = [&]() {
    int x = l;
    if constexpr (NB == 2) asm volatile("" : "+v"(x));
    return x;
  };

  // gradient entering the segment's end: dht (last segment) or the value
  // chained by pass 2; every load is issued before the first is used (null
  // reads zeros).  Gs[8 j + kb]: column block j, keys 16 kb ..
  f32x4 Gs[8 * NB];
  if (w < 4) {
    const float* src = (p == sr.p_last) ? (a.dht ? a.dht + unit * KV : nullptr)
                       : P1 ? nullptr : a.seg_start + ((int64_t)unit * a.P + p) * KV;
    const bool vf = (p == sr.p_last) && a.svf;
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(src, src ? KV * (int64_t)sizeof(float) : 0);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 16 * kb + 4 * grp + e, vc = cb0 + cw(j) + col;
          Gs[8 * j + kb][e] =
              buf_load_f32(srs, (vf ? vc * kDim + key : key * kDim + vc) * (int)sizeof(float));
        }
  }

  // wave 4's copies: per-row values and dO / A of chunk c (3 + 8 NB + 8
  // loads, in that order), q / k of chunk c (32 loads)
  float r_g = 0.f, r_gl = 0.f;
  T r_bt = from_f<T>(0.f);  // raw: converted where it is used, not where it lands
  auto chunk_rows = [&](int c) { return (int)min((int64_t)kChunk, s.end - s.start - (int64_t)kChunk * c); };
  auto issue_da = [&](int c, int lq) {
    const int bs = c & 1, Cc = chunk_rows(c);
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int gv = a.Hv * kDim * (int)sizeof(T), ga = a.Hv * kChunk * (int)sizeof(T);
    r_g = a.gcum[(t0 + min(l, Cc - 1)) * a.Hv + h];
    r_gl = a.gcum[(t0 + Cc - 1) * a.Hv + h];
    r_bt = reinterpret_cast<const T*>(a.beta)[(t0 + min(l, Cc - 1)) * a.Hv + h];
    __builtin_amdgcn_sched_barrier(0);  // the three loads first, as the waits count
    tile_dma<CW>(buf_rsrc(reinterpret_cast<const T*>(a.dO) + (t0 * a.Hv + h) * kDim + cb0,
                          (int64_t)Cc * gv),
                 gv, Ds[bs], lq);
    tile_dma<64>(buf_rsrc(reinterpret_cast<const T*>(a.A) + (t0 * a.Hv + h) * kChunk,
                          (int64_t)Cc * ga),
                 ga, As[bs], lq);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto issue_qk = [&](int c, int lq) {
    const int bs = c % 3, Cc = chunk_rows(c);
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int gq = a.Hq * kDim * (int)sizeof(T);
    tile_dma<128>(buf_rsrc(reinterpret_cast<const T*>(a.q) + (t0 * a.Hq + hq) * kDim, (int64_t)Cc * gq),
                  gq, Qs[bs], lq);
    tile_dma<128>(buf_rsrc(reinterpret_cast<const T*>(a.k) + (t0 * a.Hq + hq) * kDim, (int64_t)Cc * gq),
                  gq, Ks[bs], lq);
    __builtin_amdgcn_sched_barrier(0);
  };
  // rows past the chunk's end are zero whatever the copies left there (a
  // tile row r is bytes [r, r + 1) x its row size, swizzled within the row)
  const uint4 z4 = make_uint4(0, 0, 0, 0);
  auto zero_da = [&](int c, int l) {
    const int bs = c & 1, Cc = chunk_rows(c);
    for (int x = 16 * l; x < (kChunk - Cc) * 2 * CW; x += 1024)
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Ds[bs]) + Cc * 2 * CW + x) = z4;
    for (int x = 16 * l; x < (kChunk - Cc) * 128; x += 1024)
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(As[bs]) + Cc * 128 + x) = z4;
  };
  auto zero_qk = [&](int c, int l) {
    const int bs = c % 3, Cc = chunk_rows(c);
    for (int x = 16 * l; x < (kChunk - Cc) * 256; x += 1024) {
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Qs[bs]) + Cc * 256 + x) = z4;
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Ks[bs]) + Cc * 256 + x) = z4;
    }
  };
  auto put_rows = [&](int c, int l) {  // the per-row values loaded by issue_da(c)
    const int bs = c & 1;
    const bool ok = l < chunk_rows(c);
    const float e = __expf(r_g), r_b = to_f(r_bt);
    gam[bs][l] = r_g;
    eg[bs][l] = a.scale * e;
    bex[bs][l] = (ok ? ((OPT & 2) ? beta_used(r_b, a.beta_mode) : r_b) : 0.f) * e;
    dl[bs][l] = __expf(r_gl - r_g);
  };

  // gradient of chunk cc's end state out, packed (packed_off)
  auto dh_rsrc = [&](int cc) {
    return buf_rsrc(reinterpret_cast<T*>(a.dh) + ((choff + cc) * a.Hv + h) * KV, KV * (int64_t)sizeof(T));
  };
  // 64-column form: wave 5 stores it from the operand copies the chain left
  // in Hx; non-temporal, as this pass never reads it back (coherent, sc1,
  // when gradient workgroups in the same launch read it)
  auto store_dh = [&](int cc) {
    if constexpr (NB == 1 && !P1) {
      const __amdgpu_buffer_rsrc_t hrs = dh_rsrc(cc);
#pragma unroll
      for (int wq = 0; wq < 4; ++wq)
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) {
          const int off = packed_off(cb0 / 16 + wq, kb2, l) * (int)sizeof(T);
          const uint4 x = __builtin_bit_cast(uint4, L.Hx[wq][kb2][l]);
          if (a.flags) buf_store16_sc1(hrs, off, x);
          else buf_store16_nt(hrs, off, x);
        }
    }
  };
  // with gradient workgroups in the launch: chunk cc's state gradient is
  // complete (64-column form: this wave's stores, all issued; 128-column
  // form: the chain waves waited for theirs before the barrier this follows);
  // count it
  auto publish = [&](int cc) {
    if constexpr (NB == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    if (l == 0)
      buf_store_u32_sc1(buf_rsrc(a.flags, (int64_t)(unit * a.nvs + vs + 1) * 4),
                        (unit * a.nvs + vs) * 4, (unsigned)(nch - cc));
  };

  // before chunk c's first barrier: its q / k, dO / A and per-row values are
  // in LDS; chunk c-1's q / k copies may still be in flight
  if (w == 4 && sr.c0 < sr.c1) {
    const int cf = sr.c1 - 1;
    issue_da(cf, l);
    issue_qk(cf, l);
    if (cf - 1 >= sr.c0) {
      issue_qk(cf - 1, l);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(32));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    zero_qk(cf, l);
    zero_da(cf, l);
    put_rows(cf, l);
  }
  // the initial gradient has arrived before the loop (else the loop-entry
  // merge makes its first use wait for later loads as well)
  __builtin_amdgcn_s_waitcnt(0);
  // the two tiles above the diagonal that P^T's products read stay zero
  p_zero_tiles<T>(Ps, LDA);
  // the P tiles of waves 5, 6, 7 (3, 3, 4), (row block, column block) 4 bits
  // each: (0,0) (1,0) (1,1); (2,0) (2,1) (2,2); (3,0) (3,1) (3,2) (3,3)
  constexpr uint64_t pcode = 0x0ull | (0x4ull << 4) | (0x5ull << 8) |
                             ((0x8ull | (0x9ull << 4) | (0xAull << 8)) << 16) |
                             ((0xCull | (0xDull << 4) | (0xEull << 8) | (0xFull << 12)) << 32);
  // Wave 4 (and, in the 128-column form, the chain waves, whose state
  // gradient stores are in flight) meet the barriers without
  // __syncthreads' fences: they would wait for every copy or store in flight
  // (the LDS-direct loads count as LDS writes).  Their own waits are
  // explicit: the copies the next phase reads and the LDS stores (here); the
  // wavefront-scope fences only keep the compiler from moving memory
  // operations across the barrier.
  auto barrier = [&]() {
    if (w == 4 || (NB == 2 && w < 4)) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      __syncthreads();
    }
  };
  for (int c = sr.c1 - 1; c >= sr.c0; --c) {
    const int b = c & 1, bq = c % 3;
    barrier();  // chunk c's slots are ready; every wave is done with chunk c+1
    f32x4 dd[NB][4];
    x8 Gb[NB][4], fdo[NB][2];
    if (w == 4) {
      if (c - 1 >= sr.c0) issue_da(c - 1, fresh_lane());
    } else if (w < 4) {
      const int lq = fresh_lane();
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2)
          Gb[j][kb2] = pack_split<T>(Gs[8 * j + 2 * kb2], Gs[8 * j + 2 * kb2 + 1]);
      if constexpr (NB == 2 && !P1) {
        // chunk c+1's stores (issued an iteration ago) are complete before
        // the middle barrier, after which wave 5 counts them; then chunk c's
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        const __amdgpu_buffer_rsrc_t hrs = dh_rsrc(c);
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int kb2 = 0; kb2 < 4; ++kb2)
            buf_store16_sc1(hrs, packed_off((cb0 + cw(j)) / 16, kb2, lq) * (int)sizeof(T),
                            __builtin_bit_cast(uint4, Gb[j][kb2]));
      }
      // K dSn of chunk c in four rounds over the key dimension; every
      // fragment of a round is read before it multiplies
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) dd[j][tb] = zero4();
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        x8 fk[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) fk[tb] = frag_row_split_w<T, 128>(Ks[bq], 16 * tb, 32 * kb2, lq);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) dd[j][tb] = mfma16(fk[tb], Gb[j][kb2], dd[j][tb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // dS so far = e^{gL} dSn + Q^T (scale diag(e^gamma) dO): its dO
      // fragments, each row scaled (row 32 kt + k(grp, e) of the split order)
      const float eL = __expf(gam[b][63]);
      x8 Ob[NB][2], fr[8];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) fdo[j][kt] = frag_tr_split_w<T, CW>(Ds[b], 32 * kt, cw(j), lq);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) fr[kb] = frag_tr_split_w<T, 128>(Qs[bq], 0, 16 * kb, lq);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(eg[b] + 32 * kt + 4 * (lq >> 4));
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(eg[b] + 32 * kt + 16 + 4 * (lq >> 4));
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          x8 f = fdo[j][kt];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f[e] = from_f<T>(to_f(f[e]) * e0[e]);
            f[e + 4] = from_f<T>(to_f(f[e + 4]) * e1[e]);
          }
          Ob[j][kt] = f;
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) Gs[8 * j + kb] = mfma16(fr[kb], Ob[j][0], Gs[8 * j + kb] * eL);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) fr[kb] = frag_tr_split_w<T, 128>(Qs[bq], 32, 16 * kb, lq);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) Gs[8 * j + kb] = mfma16(fr[kb], Ob[j][1], Gs[8 * j + kb]);
    } else {
      // waves 5-7: this wave's tiles of P = lower_incl(Q K^T o Gamma) of
      // chunk c, published by the middle barrier; in the 64-column form
      // wave 5 first stores the state gradient of chunk c+1 (last in this
      // wave's vector memory queue: a later wait would also wait for these
      // stores)
      if (NB == 1 && w == 5) {
        if (a.flags && c + 2 < sr.c1) publish(c + 2);  // stored an iteration ago
        if (c + 1 < sr.c1) store_dh(c + 1);
      }
      const int sl = __builtin_amdgcn_readfirstlane(w - 5);  // wave-uniform
      const int nt = sl == 2 ? 4 : 3;
      const int lp = fresh_lane(), pgrp = lp >> 4, pcol = lp & 15;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < nt) {
          const int x = (int)((pcode >> (16 * sl + 4 * t)) & 15), rb = x >> 2, cb = x & 3;
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)  // split k order, as dh_lh_body's chain
            acc = mfma16(frag_row_split_w<T, 128>(Qs[bq], 16 * rb, 32 * kk, lp),
                         frag_row_split_w<T, 128>(Ks[bq], 16 * cb, 32 * kk, lp), acc);
          const f32x4 gr = *reinterpret_cast<const f32x4*>(gam[b] + 16 * rb + 4 * pgrp);
          const float gi = gam[b][16 * cb + pcol];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * rb + 4 * pgrp + e, i = 16 * cb + pcol;
            // masked entries take exp(-inf) = 0 (an unconditional exponential)
            const float pv = acc[e] * __expf((rb != cb || i <= r) ? gr[e] - gi : -INFINITY);
            Ps[r * LDA + i] = from_f<T>(pv);
          }
        }
      }
    }
    barrier();  // P of chunk c is in LDS; Hx is free
    if (w == 4) {
      // chunk c-2's q / k (issued here, in the chain's long phase), then
      // chunk c-1's q / k, dO / A and per-row values land before the next
      // first barrier; newer: chunk c-2's q / k (32)
      const int lq = fresh_lane();
      if (c - 2 >= sr.c0) issue_qk(c - 2, lq);
      if (c - 1 >= sr.c0) {
        if (c - 2 >= sr.c0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(32));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        zero_qk(c - 1, lq);
        zero_da(c - 1, lq);
        put_rows(c - 1, lq);
      }
      continue;
    }
    if (NB == 2 && w == 5 && a.flags && c + 1 < sr.c1) publish(c + 1);
    if (w >= 4) continue;
    // chunk c's dSn for the store wave
    if constexpr (NB == 1) {
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) L.Hx[w][kb2][l] = Gb[0][kb2];
    }

    // The products below run in rounds of independent accumulators whose
    // LDS fragments are issued before the round multiplies; the scheduling
    // fences keep the compiler from sinking every read to its product, which
    // would put one LDS latency per MFMA on the chain.
    // Fragment (tb, kt) of P^T or A^T (k = rows 32 kt ..) for kt >= tb / 2.
    auto tk = [](int tb, int kt) { return tb < 2 ? 2 * tb + kt : 2 + tb; };
    const int lq = fresh_lane();
    x8 fp[6], fa[6], fr[8];
    f32x4 dlv[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int kt = tb / 2; kt < 2; ++kt)
        fp[tk(tb, kt)] = frag_tr_split(Ps + 32 * kt * LDA + 16 * tb, LDA);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) dlv[tb] = *reinterpret_cast<const f32x4*>(dl[b] + 16 * tb + 4 * (lq >> 4));
    // dDelta = diag(e^{gL-gamma}) K dSn + scale P^T dO
    x8 Db[NB][2];
    auto delta = [&](int j, const f32x4 (&pd)[4]) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) dd[j][tb][e] = dlv[tb][e] * dd[j][tb][e] + a.scale * pd[tb][e];
      Db[j][0] = pack_split<T>(dd[j][0], dd[j][1]);
      Db[j][1] = pack_split<T>(dd[j][2], dd[j][3]);
    };
    if constexpr (NB == 1) {
      __builtin_amdgcn_sched_barrier(0);
      f32x4 pd[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) pd[tb] = zero4();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          if (kt >= tb / 2) pd[tb] = mfma16(fp[tk(tb, kt)], fdo[0][kt], pd[tb]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int kt = tb / 2; kt < 2; ++kt)
          fa[tk(tb, kt)] = frag_tr_split_w<T, 64>(As[b], 32 * kt, 16 * tb, lq);
      __builtin_amdgcn_sched_barrier(0);
      delta(0, pd);
    } else {
      // 128-column form: one column block at a time, its dO fragments read
      // again (chunk c's slot is unchanged until the next iteration's
      // copies) rather than held across the barrier
      x8 fo[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) fo[0][kt] = frag_tr_split_w<T, CW>(Ds[b], 32 * kt, cw(0), lq);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) fo[1][kt] = frag_tr_split_w<T, CW>(Ds[b], 32 * kt, cw(1), lq);
      f32x4 pd[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) pd[tb] = zero4();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          if (kt >= tb / 2) pd[tb] = mfma16(fp[tk(tb, kt)], fo[0][kt], pd[tb]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int kt = tb / 2; kt < 2; ++kt)
          fa[tk(tb, kt)] = frag_tr_split_w<T, 64>(As[b], 32 * kt, 16 * tb, lq);
      delta(0, pd);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) pd[tb] = zero4();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          if (kt >= tb / 2) pd[tb] = mfma16(fp[tk(tb, kt)], fo[1][kt], pd[tb]);
      __builtin_amdgcn_sched_barrier(0);
      delta(1, pd);
    }
    // Z = -diag(beta e^gamma) A^T dDelta
    f32x4 zz[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) zz[j][tb] = zero4();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          if (kt >= tb / 2) zz[j][tb] = mfma16(fa[tk(tb, kt)], Db[j][kt], zz[j][tb]);
    // dS += K^T Z
    x8 Zb[NB][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const f32x4 bx = *reinterpret_cast<const f32x4*>(bex[b] + 16 * tb + 4 * (lq >> 4));
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) zz[j][tb][e] *= -bx[e];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      Zb[j][0] = pack_split<T>(zz[j][0], zz[j][1]);
      Zb[j][1] = pack_split<T>(zz[j][2], zz[j][3]);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) fr[kb] = frag_tr_split_w<T, 128>(Ks[bq], 32 * kt, 16 * kb, lq);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) Gs[8 * j + kb] = mfma16(fr[kb], Zb[j][kt], Gs[8 * j + kb]);
    }
  }

  // the dSn of the last chunk walked (c0): 64-column form, wave 5 stores it;
  // 128-column form, the chain's own stores are complete before the barrier
  if (NB == 2 && w < 4) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  if (w == 5 && sr.c0 < sr.c1) {
    if (NB == 1) {
      if (a.flags && sr.c0 + 1 < sr.c1) publish(sr.c0 + 1);
      store_dh(sr.c0);
    }
    if (a.flags) publish(sr.c0);
  }
  if (w >= 4) return;
  if (P1) {
    float* so = a.seg_out + ((int64_t)unit * a.P + p) * (2 * KV);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          so[(16 * kb + 4 * grp + e) * (2 * kDim) + kDim + cb0 + cw(j) + col] = Gs[8 * j + kb][e];
  } else if (p == 0 && a.dh0) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 16 * kb + 4 * grp + e, vc = cb0 + cw(j) + col;
          a.dh0[unit * KV + (a.svf ? vc * kDim + key : key * kDim + vc)] = Gs[8 * j + kb][e];
        }
  } else if (a.sliced && p > 0) {
    // the gradient entering the previous segment's end, for the next launch
    float* dst = a.seg_next + ((int64_t)unit * a.P + p - 1) * KV;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[(16 * kb + 4 * grp + e) * kDim + cb0 + cw(j) + col] = Gs[8 * j + kb][e];
  }
}

// The output passes of B1 and B2 with load-helper waves (VB = 1), in one
// launch of 8-wave workgroups: blocks [0, n1) take B1.
template <typename T, int OPT>
__global__ __launch_bounds__(512) void bwd_scans_lh_kernel(ScanArgs sa, DhArgs da, int n1) {
  __shared__ DhLhLds<T> lds;
  if ((int)blockIdx.x < n1) scan_spec_body<T, MODE_STATE, OPT>(sa, (int)blockIdx.x, n1);
  else dh_lh_body<T, OPT>(da, (int)blockIdx.x - n1, (int)gridDim.x - n1, lds);
}

// The state-gradient scan's output pass alone (the forward's states given,
// q / k not normalised in the kernel): the loader-wave form.
template <typename T, int OPT>
__global__ __launch_bounds__(512) void dh_ld_kernel(DhArgs da) {
  __shared__ DhLdLds<T> lds;
  dh_ld_body<T, OPT>(da, (int)blockIdx.x, (int)gridDim.x, lds);
}

// The same at two tiles per wave: one 128-column workgroup per unit and
// segment (the body of the data-scheduled launch's scan, without the
// progress counts); OPT bit 2 runs pass 1 of a split backward.
template <typename T, int OPT>
__global__ __launch_bounds__(512) void dh_ld2_kernel(DhArgs da) {
  __shared__ DhLdLds<T, 2> lds;
  dh_ld_body<T, OPT, 2, (OPT & 4) ? 5 : 4>(da, (int)blockIdx.x, (int)gridDim.x, lds);
}

// Pass 1 of the state-gradient scan alone (the forward's states given): with
// no state-scan LDS beside it two workgroups fit a CU at VB = 1.
template <typename T, int VB>
__global__ __launch_bounds__(256, VB == 1 ? 2 : 1) void dh_aug_kernel(DhArgs da) {
  dh_body<T, VB, MODE_AUG>(da, (int)blockIdx.x, (int)gridDim.x);
}

// The state scan (B1) and the state-gradient scan (B2) are independent (B2
// needs no chunk states), so one launch runs both: blocks [0, n1) take B1,
// the rest B2.  Each pass alone fills only part of the chip when there are
// few (sequence, head) units.
template <typename T, int VB, int MS, int MD>
__global__ __launch_bounds__(256, 1) void bwd_scans_kernel(ScanArgs sa, DhArgs da, int n1) {
  if ((int)blockIdx.x < n1) scan_body<T, VB, MS>(sa, (int)blockIdx.x, n1);
  else dh_body<T, VB, MD>(da, (int)blockIdx.x - n1, (int)gridDim.x - n1);
}

// ---------------------------------------------------------------------------
// B3-B5: per-chunk gradients
// ---------------------------------------------------------------------------
struct GradArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  const void* beta;
  const float* gcum;
  const void* A;
  const void* h;   // [NC, Hv] packed chunk-start states (packed_off)
  const void* dh;  // [NC, Hv] packed end-state gradients
  void* dq;        // in_dtype [T, Hq, K]
  void* dk;
  void* dv;
  void* dbeta;
  void* dg;
  const int32_t* cu;
  const int32_t* offs;
  int N, T, Hq, Hv, nc_dense, g_dtype;
  float scale;
  float* gacc;    // GVA: [G - 1 heads][NC, Hq, 8 waves, 8, 64 lanes, 4] fp32 dq / dk rows
  int gva_final;  // GVA: 0 the launch of heads 0 .. G-2, 1 the launch of head G-1
  // a pipelined slice of a dense batch (sl_len > 0): workgroup row x takes
  // chunk sl_c0 + x % sl_len of sequence x / sl_len
  int sl_c0, sl_len;
  int qk_norm;    // q, k rows scaled to unit length before use
  // (qk_norm) the rows were normalised beforehand: q and k hold the unit
  // rows, and these their 1 / |x| per (token, q head) row; else null
  const float* qinv;
  const float* kinv;
  int beta_mode;  // bit 0 sigmoid of a beta logit, bit 1 twice beta
  // the gate (use_gate): g is the gate input graw, dg is with respect to it,
  // and each workgroup leaves its chunk's shares of the parameter gradients
  // (sum of dlogdecay * logdecay, sum of dg) in gpart[(c * Hv + h) * 2 + {0, 1}]
  const void* graw;
  const float* gate_A_log;  // non-null iff the gate is on
  const float* gate_dt_bias;
  float* gpart;
  // the state gradients are being written in the same launch (bwd_dyn_kernel):
  // load them coherently (sc1); the progress counts a workgroup waits for
  const unsigned* flags;
  // (bwd_dyn_kernel, packed sequences) the gradient items in launch order:
  // (sequence, chunk) pairs (dyn_items_kernel)
  const int32_t* items;
};

// Eight waves: wave w works on row / column block wr = w % 4 and takes one
// side of every phase (hi = w / 4): hi = 0 the forward-side chain (K S, R,
// Delta, dP, dQ1 = dO S^T and everything of dq), hi = 1 the gradient side
// (K dSn, dDelta, dR, dX = -dR S^T, dKs = Delta dSn^T, dM = -dR Delta^T and
// everything of dk).  The two sides of a phase are independent, so two waves share each
// SIMD and hide each other's latencies.
// A workgroup takes one (chunk, value head).  With GVA (Hq < Hv) the kernel
// runs twice: the first launch takes value heads 0 .. G-2 of every group and
// leaves each head's dq, dk contribution in its fp32 workspace slot; the
// second takes head G-1, adds the slots in head order to its own
// contribution and stores dq, dk (the kernel boundary orders the two).
// LDS of one gradient workgroup (grad_body), a struct so that a launch can
// share its LDS with another pass's workgroups.
template <typename T>
struct GradLds {
  // 64-wide tiles: row stride 72 elements (36 banks) for the tiles read as
  // row operands as often as transposed, 80 (40 banks) for those read
  // mostly by the transposing loads (P, V, dO, Delta, dR).  A transposing
  // load takes 32 bytes of four consecutive rows per 16 lanes; at 40 banks
  // per row those land on distinct banks (at 36 they overlap two ways).
  static constexpr int L7 = 72;
  static constexpr int LT = 80;
  alignas(16) T Qs[QK_TILE];  // q, k, S^T, dSn^T: staggered rows (qk_row)
  alignas(16) T Ks[QK_TILE];
  alignas(16) T As[64 * L7];
  alignas(16) T Ps[64 * LT];
  alignas(16) T Ss[QK_TILE];    // S[:, half]^T ([v][k]); later dq (ld LD)
  alignas(16) T Gs_[QK_TILE];   // dSn[:, half]^T; later dP o Gamma, dM o beta Gamma, dk
  alignas(16) T Vs[64 * LT];
  alignas(16) T Os[64 * LT];    // dO[:, half]
  alignas(16) T Dls[64 * LT];   // Delta, transposed
  alignas(16) T DRs[64 * LT];   // dR, transposed
  alignas(16) T DVs[64 * L7];   // dv of the half, row-major
  alignas(16) float gam[64];
  alignas(16) float bet[64];
  alignas(16) float eg[64];
  alignas(16) float bex[64];
  alignas(16) float dl[64];
  alignas(16) float dbv[8][64];     // v . dR partials per (half, column block)
  alignas(16) float colE[4][64];    // column sums of dP o P per row block
  alignas(16) float colE2[4][64];   // column sums of dM o M per row block
  alignas(16) float red[8];         // <S, dSn> per wave
  alignas(16) float dgam[64];
  alignas(16) float fsum[4][4];     // F partials per (row block, lane group)
  alignas(16) float rowq[64];       // dgamma row terms of the dq side
  alignas(16) float dbf[64];        // d beta / d (beta input) per row
  alignas(16) float xinv[2][64];    // 1 / |q|, 1 / |k| per row (q / k normalisation)
  alignas(16) float gsl[2][64];     // the gate's slope and log decay per row (gate on)
};

// What a gradient workgroup loads first: the q, k and A tiles, the per-row
// values and value half 0's tiles (the half's registers serve half 1 after).
template <typename T>
struct GradFirst {
  TileRegs<128, 512> rq, rk, rs, rg;
  TileRegs<64, 512> ra, rv, ro;
  float gr = 0.f, gl = 0.f;
  T b = from_f<T>(0.f);
  uint32_t x = 0;  // raw bits of the gate input
};

// An item's place: global chunk row c, its sequence n and first token t0,
// its valid rows Cc, the q / k head hq and the value head h (gr: h's index
// in its group).
struct GradItem {
  int c, n;
  int64_t t0;
  int Cc, hq, gr, h;
};

template <bool GVA>
__device__ __forceinline__ GradItem grad_item(const GradArgs& a, int c, int by) {
  GradItem it;
  if (a.sl_len > 0) c = (c / a.sl_len) * a.nc_dense + a.sl_c0 + c % a.sl_len;
  int j;
  if (a.cu) {
    it.n = find_seq(a.offs, a.N, c);
    j = c - a.offs[it.n];
  } else {
    it.n = c / a.nc_dense;
    j = c % a.nc_dense;
  }
  const SeqInfo s = seq_info(a.cu, it.n, a.T);
  it.c = c;
  it.t0 = s.start + (int64_t)kChunk * j;
  it.Cc = (int)min((int64_t)kChunk, s.end - it.t0);
  const int G = a.Hv / a.Hq;
  // GVA: the first launch has (G - 1) x Hq rows of workgroups (head r of
  // group hq at row hq * (G - 1) + r), the second (gva_final) Hq rows
  it.hq = !GVA ? by / G : a.gva_final ? by : by / (G - 1);
  it.gr = !GVA ? 0 : a.gva_final ? G - 1 : by % (G - 1);
  it.h = GVA ? it.hq * G + it.gr : by;
  return it;
}

// The loads of a value half's tiles: S^T, dSn^T (packed, 16 KiB each) and
// the half's V and dO columns.
// The state gradient's half (dSn^T, packed): coherent loads (sc1) when the
// state gradients are written in the same launch.
template <typename T>
__device__ __forceinline__ void grad_dsn_load(const GradArgs& a, const GradItem& it, int v0,
                                              TileRegs<128, 512>& rg) {
  const int64_t KV = (int64_t)kDim * kDim;
  const T* hG = reinterpret_cast<const T*>(a.dh) + ((int64_t)it.c * a.Hv + it.h) * KV;
  if (a.flags) tile_load<T, 128, 512, 16>(rg, hG + v0 * kDim, kDim, 64);
  else tile_load<T, 128, 512>(rg, hG + v0 * kDim, kDim, 64);
}

// with_dsn false: every tile of the half but the state gradient's
template <typename T>
__device__ __forceinline__ void grad_half_loads(const GradArgs& a, const GradItem& it, int v0,
                                                TileRegs<128, 512>& rs, TileRegs<128, 512>& rg,
                                                TileRegs<64, 512>& rv, TileRegs<64, 512>& ro,
                                                bool with_dsn = true) {
  const int64_t KV = (int64_t)kDim * kDim;
  const T* hS = reinterpret_cast<const T*>(a.h) + ((int64_t)it.c * a.Hv + it.h) * KV;
  tile_load<T, 128, 512>(rs, hS + v0 * kDim, kDim, 64);
  if (with_dsn) grad_dsn_load<T>(a, it, v0, rg);
  tile_load<T, 64, 512>(rv, reinterpret_cast<const T*>(a.v) + (it.t0 * a.Hv + it.h) * kDim + v0,
                        (int64_t)a.Hv * kDim, it.Cc);
  tile_load<T, 64, 512>(ro, reinterpret_cast<const T*>(a.dO) + (it.t0 * a.Hv + it.h) * kDim + v0,
                        (int64_t)a.Hv * kDim, it.Cc);
}

// The first loads of an item: q, k, A, the per-row values (threads 0..63),
// then value half 0 (with_dsn false: without its state gradient).
template <typename T>
__device__ __forceinline__ void grad_first_loads(const GradArgs& a, const GradItem& it,
                                                 GradFirst<T>& f, bool with_dsn = true) {
  const int tid = threadIdx.x;
  tile_load<T, 128, 512>(f.rq, reinterpret_cast<const T*>(a.q) + (it.t0 * a.Hq + it.hq) * kDim,
                         (int64_t)a.Hq * kDim, it.Cc);
  tile_load<T, 128, 512>(f.rk, reinterpret_cast<const T*>(a.k) + (it.t0 * a.Hq + it.hq) * kDim,
                         (int64_t)a.Hq * kDim, it.Cc);
  tile_load<T, 64, 512>(f.ra, reinterpret_cast<const T*>(a.A) + (it.t0 * a.Hv + it.h) * kChunk,
                        (int64_t)a.Hv * kChunk, it.Cc);
  if (tid < 64) {
    const int64_t row = (it.t0 + min(tid, it.Cc - 1)) * a.Hv + it.h;
    f.gr = a.gcum[row];
    f.gl = a.gcum[(it.t0 + it.Cc - 1) * a.Hv + it.h];
    f.b = reinterpret_cast<const T*>(a.beta)[row];
    if (a.gate_A_log)  // raw bits: converted after the tile stores
      f.x = a.g_dtype == 2 ? reinterpret_cast<const uint32_t*>(a.graw)[row]
                           : (uint32_t)reinterpret_cast<const uint16_t*>(a.graw)[row];
  }
  grad_half_loads<T>(a, it, 0, f.rs, f.rg, f.rv, f.ro, with_dsn);
}

// One (chunk row c, workgroup row by) of the gradient pass; nbx is the
// number of chunk rows of the launch (the GVA slots' stride).  f receives the
// item's first loads (grad_first_loads); PRE: the caller has issued them.
template <typename T, bool QKN, bool GVA, bool PRE = false>
__device__ __forceinline__ void grad_body(const GradArgs& a, int c, int by, int nbx,
                                          GradLds<T>& L, GradFirst<T>& f) {
  const GradItem item = grad_item<GVA>(a, c, by);
  c = item.c;
  typedef typename VT<T>::x8 x8;
  constexpr int LD = 136;  // row stride of the dq / dk staging in Ss / Gs_
  constexpr int L7 = GradLds<T>::L7, LT = GradLds<T>::LT;
  auto& Qs = L.Qs;
  auto& Ks = L.Ks;
  auto& As = L.As;
  auto& Ps = L.Ps;
  auto& Ss = L.Ss;
  auto& Gs_ = L.Gs_;
  auto& Vs = L.Vs;
  auto& Os = L.Os;
  auto& Dls = L.Dls;
  auto& DRs = L.DRs;
  auto& DVs = L.DVs;
  auto& gam = L.gam;
  auto& bet = L.bet;
  auto& eg = L.eg;
  auto& bex = L.bex;
  auto& dl = L.dl;
  auto& dbv = L.dbv;
  auto& colE = L.colE;
  auto& colE2 = L.colE2;
  auto& red = L.red;
  auto& dgam = L.dgam;
  auto& fsum = L.fsum;
  auto& rowq = L.rowq;
  auto& dbf = L.dbf;
  auto& xinv = L.xinv;
  auto& gsl = L.gsl;
  // side 1's row terms of the last step (rowacc, k . dX, F, dbeta part), in
  // the P tile's storage (dead once the value halves are done)
  float* const rowv = reinterpret_cast<float*>(Ps);

  const int64_t t0 = item.t0;
  const int Cc = item.Cc;
  const int G = a.Hv / a.Hq;
  const int hq = item.hq, gr = item.gr, h = item.h;
  const bool store_dqk = !GVA || a.gva_final;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;
  const int wr = w & 3;
  const bool hi = w >= 4;

  // the value-half tiles: S^T, dSn^T (value-major LDS rows v0 .. v0+63) and
  // V, dO (columns v0 .. v0+63); half 1 is prefetched while half 0 computes
  TileRegs<128, 512>& rs = f.rs;
  TileRegs<128, 512>& rg = f.rg;
  TileRegs<64, 512>& rv = f.rv;
  TileRegs<64, 512>& ro = f.ro;
  auto load_half = [&](int v0) { grad_half_loads<T>(a, item, v0, rs, rg, rv, ro); };
  // (the states are packed: the half's 16 KiB load in storage order and
  // scatter into value-major LDS rows)
  float sds = 0.f;
  auto store_half = [&]() {
#pragma unroll
    for (int i = 0; i < TileRegs<128, 512>::N; ++i) sds += dot8<T>(rs.r[i], rg.r[i]);
    tile_store_packed_q<T, 512>(Ss, rs);
    tile_store_packed_q<T, 512>(Gs_, rg);
    tile_store<T, 64, 512>(Vs, LT, rv);
    tile_store<T, 64, 512>(Os, LT, ro);
  };
  // q, k, A and the per-row values (gamma, beta, the gate input) are loaded
  // and stored first; value half 0's tiles (S^T, dSn^T, V, dO) are issued
  // next and stored only after the P / N phase, which overlaps their latency
  if (!PRE) grad_first_loads<T>(a, item, f);
  {
    if (QKN) {
      if (a.qinv) {  // unit rows given: their 1 / |x|
        if (tid < 64) {
          const int64_t row = (t0 + min(tid, Cc - 1)) * a.Hq + hq;
          xinv[0][tid] = a.qinv[row];
          xinv[1][tid] = a.kinv[row];
        }
      } else {
        l2norm_rows<T, 512>(f.rq, xinv[0]);
        l2norm_rows<T, 512>(f.rk, xinv[1]);
      }
    }
    tile_store_q<T, 512>(Qs, f.rq);
    tile_store_q<T, 512>(Ks, f.rk);
    tile_store<T, 64, 512>(As, L7, f.ra);
  }
  const uint32_t p_x = f.x;
  if (tid < 64) {
    const float gr = f.gr, gl = f.gl, bx = to_f(f.b);
    const float bt = (tid < Cc) ? beta_used(bx, a.beta_mode) : 0.f;
    const float e = __expf(gr);
    gam[tid] = gr;
    bet[tid] = bt;
    dbf[tid] = beta_used_grad(bx, a.beta_mode);
    eg[tid] = e;
    bex[tid] = bt * e;
    dl[tid] = __expf(gl - gr);
    dgam[tid] = 0.f;
    if (a.gate_A_log) {
      const float ga = a.gate_A_log[h], gb = a.gate_dt_bias ? a.gate_dt_bias[h] : 0.f;
      const float xin = a.g_dtype == 2 ? __builtin_bit_cast(float, p_x)
                        : a.g_dtype == 0 ? __builtin_bit_cast(float, p_x << 16)
                                         : (float)__builtin_bit_cast(_Float16, (uint16_t)p_x);
      gsl[0][tid] = tid < Cc ? gate_log_decay_grad(xin, ga, gb) : 0.f;
      gsl[1][tid] = tid < Cc ? gate_log_decay(xin, ga, gb) : 0.f;
    }
  }
  __syncthreads();

  // rows 16 wr .. 16 wr + 15 of P = lower_incl(Q K^T o Gamma) (side 0, also
  // written to Ps) or N = strict_lower(K K^T o Gamma) (side 1), fp32
  f32x4 pn[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    f32x4 acc = zero4();
    if (cb <= wr) {
      const T* rows = hi ? Ks : Qs;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma16(frag_row_q(rows, 16 * wr, 32 * kk), frag_row_q(Ks, 16 * cb, 32 * kk), acc);
    }
    const f32x4 gr = *reinterpret_cast<const f32x4*>(gam + 16 * wr + 4 * grp);
    const float gi = gam[16 * cb + col];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * wr + 4 * grp + e, i = 16 * cb + col;
      const bool keep = hi ? (i < r) : (i <= r);
      // masked by a select, not a zero factor: for cb > wr, acc is defined
      // only if the compiler branches around the products above (an MFMA
      // does not honour the EXEC mask)
      pn[cb][e] = keep ? acc[e] * __expf(gr[e] - gi) : 0.f;
      if (!hi) Ps[r * LT + i] = from_f<T>(pn[cb][e]);
    }
  }

  // half 0's tiles; the barrier also publishes Ps, which side 1 reads below
  store_half();
  __syncthreads();

  // accumulators over the value halves: side 0 accB = dP, acc1 = dQ1;
  // side 1 accM = dR Delta^T, acc1 = dX, acc2 = dKs.  dR Delta^T is
  // A^T dA A^T: with Delta = A R and dA = dDelta R^T,
  // A^T dDelta R^T A^T = (A^T dDelta)(A R)^T = dR Delta^T, so
  // dM = strict_lower(-dR Delta^T) needs neither dA nor R.
  f32x4 accM[4], accB[4], acc1[8], acc2[8];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    accM[x] = zero4();
    accB[x] = zero4();
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    acc1[x] = zero4();
    acc2[x] = zero4();
  }
  // unrolled: a shared body would give half 1's prefetched tiles the
  // registers of half 0's products, so half 0 would wait for the prefetch
  // to land and copy it aside first
#pragma unroll
  for (int hv = 0; hv < 2; ++hv) {
    const int v0 = 64 * hv;
    if (hv > 0) {
      __syncthreads();  // every wave is done with the previous half's tiles
      store_half();
      __syncthreads();
    } else {
      load_half(64);  // in flight during half 0
    }

    // ---- value columns cc .. cc+15 of this half ----
    const int cc = 16 * wr;
    if (!hi) {
      // R = diag(beta) V - diag(beta e^gamma) K S ; Delta = A R
      f32x4 ks[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) ks[tb] = zero4();
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        const x8 fs = frag_row_split_q(Ss, cc, 32 * kb2);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          ks[tb] = mfma16(frag_row_split_q(Ks, 16 * tb, 32 * kb2), fs, ks[tb]);
      }
      f32x4 R[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const f32x4 vd = frag_d4(Vs, LT, 16 * tb, cc);
        const f32x4 bt = *reinterpret_cast<const f32x4*>(bet + 16 * tb + 4 * grp);
        const f32x4 bx = *reinterpret_cast<const f32x4*>(bex + 16 * tb + 4 * grp);
#pragma unroll
        for (int e = 0; e < 4; ++e) R[tb][e] = bt[e] * vd[e] - bx[e] * ks[tb][e];
      }
      const x8 Rb0 = pack_split<T>(R[0], R[1]), Rb1 = pack_split<T>(R[2], R[3]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 acc = mfma16(frag_row_split(As + 16 * tb * L7, L7), Rb0, zero4());
        if (tb >= 2) acc = mfma16(frag_row_split(As + 16 * tb * L7 + 32, L7), Rb1, acc);
        store_d4_t<T>(Dls, LT, 16 * tb, cc, acc);
      }
    } else {
      // dDelta = diag(e^{gL-gamma}) K dSn + scale P^T dO ; dR = A^T dDelta
      f32x4 kg[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) kg[tb] = zero4();
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        const x8 fg = frag_row_split_q(Gs_, cc, 32 * kb2);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          kg[tb] = mfma16(frag_row_split_q(Ks, 16 * tb, 32 * kb2), fg, kg[tb]);
      }
      f32x4 dD[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 pt = zero4();
#pragma unroll
        for (int kt = tb / 2; kt < 2; ++kt)
          pt = mfma16(frag_tr_split(Ps + 32 * kt * LT + 16 * tb, LT),
                      frag_tr_split(Os + 32 * kt * LT + cc, LT), pt);
        const f32x4 dlr = *reinterpret_cast<const f32x4*>(dl + 16 * tb + 4 * grp);
#pragma unroll
        for (int e = 0; e < 4; ++e) dD[tb][e] = dlr[e] * kg[tb][e] + a.scale * pt[e];
      }
      const x8 Db0 = pack_split<T>(dD[0], dD[1]), Db1 = pack_split<T>(dD[2], dD[3]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f32x4 dR = mfma16(frag_tr_split(As + 32 * L7 + 16 * tb, L7), Db1, zero4());
        if (tb < 2) dR = mfma16(frag_tr_split(As + 16 * tb, L7), Db0, dR);
        // the v . dR part of dbeta, and dv = diag(beta) dR
        const f32x4 vd = frag_d4(Vs, LT, 16 * tb, cc);
        const f32x4 bt = *reinterpret_cast<const f32x4*>(bet + 16 * tb + 4 * grp);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tb + 4 * grp + e;
          const float pdot = sum16(vd[e] * dR[e]);
          if (col == 0) dbv[4 * hv + wr][r] = pdot;
          DVs[r * L7 + cc + col] = from_f<T>(bt[e] * dR[e]);
        }
        store_d4_t<T>(DRs, LT, 16 * tb, cc, dR);
      }
    }
    __syncthreads();
    tile_from_lds<T, 64, 512, true>(reinterpret_cast<T*>(a.dv) + (t0 * a.Hv + h) * kDim + v0,
                              (int64_t)a.Hv * kDim, DVs, L7, Cc);

    // ---- rows 16 wr .. 16 wr + 15, contractions over this half's v ----
#pragma unroll
    for (int vk = 0; vk < 2; ++vk) {
      if (!hi) {
        const x8 fdo = frag_row_split(Os + 16 * wr * LT + 32 * vk, LT);
        // all four column blocks: the blocks above the diagonal are masked
        // by selects later (an MFMA alone under a per-wave condition would
        // run regardless of EXEC, on operands never loaded)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
          accB[ib] = mfma16(fdo, frag_tr_split(Dls + 32 * vk * LT + 16 * ib, LT), accB[ib]);
        // two rounds of four key blocks, fragments read before the products
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          x8 fs4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) fs4[i] = frag_tr_split_q(Ss, 32 * vk, 16 * (4 * kh + i));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc1[4 * kh + i] = mfma16(fdo, fs4[i], acc1[4 * kh + i]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        const x8 fdr = frag_tr_split(DRs + 32 * vk * LT + 16 * wr, LT);
        const x8 fdl = frag_tr_split(Dls + 32 * vk * LT + 16 * wr, LT);
        // dR Delta^T, all four column blocks (masked by selects later)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
          accM[ib] = mfma16(fdr, frag_tr_split(Dls + 32 * vk * LT + 16 * ib, LT), accM[ib]);
        // four rounds of two key blocks, each round's fragments read before
        // its four independent products issue
#pragma unroll
        for (int kh = 0; kh < 4; ++kh) {
          x8 fs2[2], fg2[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            fs2[i] = frag_tr_split_q(Ss, 32 * vk, 16 * (2 * kh + i));
            fg2[i] = frag_tr_split_q(Gs_, 32 * vk, 16 * (2 * kh + i));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            acc1[2 * kh + i] = mfma16(fdr, fs2[i], acc1[2 * kh + i]);
            acc2[2 * kh + i] = mfma16(fdl, fg2[i], acc2[2 * kh + i]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
  // <S, dSn>: wave sums, then the eight wave partials in a fixed order
  {
    const float x = sum4g(sum16(sds));
    if (l == 0) red[w] = x;
  }
  __syncthreads();

  // ---- C x C terms, rows r = 16 wr + 4 grp + e ----
  // side 0: dP (masked, scaled) -> dP o Gamma and the E = dP o P row / column
  // sums; side 1: dM = strict_lower(-dR Delta^T) -> dM o beta Gamma, the
  // E2 = dM o M row / column sums and the dbeta row terms (M = beta_r N,
  // N = (k_r . k_i) Gamma_ri, the side's pn)
  T* dPG = Gs_;             // bf16 dP o Gamma
  T* DMs = Gs_ + 64 * L7;   // bf16 dM o beta Gamma
  float rowacc[4] = {0.f, 0.f, 0.f, 0.f};  // dgamma row terms (E on side 0, E2 on side 1)
  float dbacc[4] = {0.f, 0.f, 0.f, 0.f};   // dbeta row terms (side 1)
  {
    const f32x4 gr = *reinterpret_cast<const f32x4*>(gam + 16 * wr + 4 * grp);
    const f32x4 br = *reinterpret_cast<const f32x4*>(bet + 16 * wr + 4 * grp);
    float gis[4];  // gamma of each column block's column, read at once
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) gis[cb] = gam[16 * cb + col];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      float cs = 0.f;
      const float gi = gis[cb];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * wr + 4 * grp + e, i = 16 * cb + col;
        if (!hi) {
          const bool keep = i <= r;
          const float dpv = keep ? a.scale * accB[cb][e] : 0.f;
          const float E = dpv * pn[cb][e];
          rowacc[e] += E;
          cs += E;
          dPG[r * L7 + i] = from_f<T>(dpv * __expf(keep ? gr[e] - gi : -INFINITY));
        } else {
          const bool keep = i < r;
          const float dm = keep ? -accM[cb][e] : 0.f;
          dbacc[e] += dm * pn[cb][e];
          const float E2 = dm * br[e] * pn[cb][e];
          rowacc[e] += E2;
          cs += E2;
          DMs[r * L7 + i] = from_f<T>(dm * br[e] * __expf(keep ? gr[e] - gi : -INFINITY));
        }
      }
      cs = sum4g(cs);
      if (grp == 0) (hi ? colE2 : colE)[wr][16 * cb + col] = cs;
    }
  }
  __syncthreads();
  // dgamma -= column sums of dP o P and of dM o M (fixed order over row blocks)
  if (tid < 64)
    dgam[tid] -= (colE[0][tid] + colE[1][tid] + colE[2][tid] + colE[3][tid]) +
                 (colE2[0][tid] + colE2[1][tid] + colE2[2][tid] + colE2[3][tid]);
  // side 0: dQ2 = (dP o Gamma) K; side 1: dK2 = (dP o Gamma)^T Q (dK3 below)
  f32x4 acc3[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) acc3[x] = zero4();
  if (!hi) {
#pragma unroll
    for (int ik = 0; ik < 2; ++ik) {
      const x8 fa = frag_row_split(dPG + 16 * wr * L7 + 32 * ik, L7);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        acc3[kb] = mfma16(fa, frag_tr_split_q(Ks, 32 * ik, 16 * kb), acc3[kb]);
    }
  } else {
#pragma unroll
    for (int ik = 0; ik < 2; ++ik) {
      const x8 fb = frag_tr_split(dPG + 32 * ik * L7 + 16 * wr, L7);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        acc3[kb] = mfma16(fb, frag_tr_split_q(Qs, 32 * ik, 16 * kb), acc3[kb]);
    }
  }

  // ---- final rows ----
  float rs1[4] = {0.f, 0.f, 0.f, 0.f}, rs2[4] = {0.f, 0.f, 0.f, 0.f};
  float dxv[8][4];
  if (hi) {
    // dK3 = D K + D^T K with D = dM o beta Gamma
#pragma unroll
    for (int ik = 0; ik < 2; ++ik) {
      const x8 fa = frag_row_split(DMs + 16 * wr * L7 + 32 * ik, L7);
      const x8 fb = frag_tr_split(DMs + 32 * ik * L7 + 16 * wr, L7);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const x8 fk = frag_tr_split_q(Ks, 32 * ik, 16 * kb);
        acc3[kb] = mfma16(fa, fk, acc3[kb]);
        acc3[kb] = mfma16(fb, fk, acc3[kb]);
      }
    }
    // dk = dK2 + dK3 + diag(e^{gL-gamma}) dKs + diag(beta e^gamma) dX, with
    // dX = -dR S^T; row sums k . dX (rs1) and k . dKs (rs2)
    const f32x4 dlr = *reinterpret_cast<const f32x4*>(dl + 16 * wr + 4 * grp);
    const f32x4 bxr = *reinterpret_cast<const f32x4*>(bex + 16 * wr + 4 * grp);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f32x4 kd = frag_d4_q(Ks, 16 * wr, 16 * kb);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dx = -acc1[kb][e];
        rs1[e] += kd[e] * dx;
        rs2[e] += kd[e] * acc2[kb][e];
        dxv[kb][e] = acc3[kb][e] + dlr[e] * acc2[kb][e] + bxr[e] * dx;
      }
    }
  } else {
    // dq = scale diag(e^gamma) dQ1 + dQ2; row sums q . dQ1 (rs1)
    const f32x4 er = *reinterpret_cast<const f32x4*>(eg + 16 * wr + 4 * grp);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f32x4 qd = frag_d4_q(Qs, 16 * wr, 16 * kb);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rs1[e] += qd[e] * acc1[kb][e];
        dxv[kb][e] = a.scale * er[e] * acc1[kb][e] + acc3[kb][e];
      }
    }
  }
  // GVA: the group sum over the value heads, in head order.  Each head but
  // the last leaves its rows in its fp32 workspace slot (register order:
  // element kb of lane l at float4 kb * 64 + l, so each store is 1 KiB
  // contiguous); the last adds the slots, head 0 first, to its own rows.
  if (GVA) {
    const int64_t slot = (int64_t)nbx * a.Hq * 8 * 512;  // float4s per head slot
    f32x4* acc = reinterpret_cast<f32x4*>(a.gacc) + (((int64_t)c * a.Hq + hq) * 8 + w) * 512 + l;
    if (a.gva_final) {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        f32x4 sum = acc[kb * 64];
        for (int rr = 1; rr < G - 1; ++rr) sum += acc[rr * slot + kb * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) dxv[kb][e] = sum[e] + dxv[kb][e];
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
        acc[gr * slot + kb * 64] = f32x4{dxv[kb][0], dxv[kb][1], dxv[kb][2], dxv[kb][3]};
    }
  }
  // With q / k normalisation dxv is the gradient with respect to the unit
  // rows x^ (q^ on side 0, k^ on side 1); the raw rows' gradient is
  // (dxv - x^ (x^ . dxv)) / |x| (on the group sum: the map is linear).
  if (QKN && store_dqk) {
    const T* X = hi ? Ks : Qs;
    float dot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f32x4 xd = frag_d4_q(X, 16 * wr, 16 * kb);
#pragma unroll
      for (int e = 0; e < 4; ++e) dot[e] += xd[e] * dxv[kb][e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) dot[e] = sum16(dot[e]);
    const f32x4 ri = *reinterpret_cast<const f32x4*>(xinv[hi ? 1 : 0] + 16 * wr + 4 * grp);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const f32x4 xd = frag_d4_q(X, 16 * wr, 16 * kb);
#pragma unroll
      for (int e = 0; e < 4; ++e) dxv[kb][e] = ri[e] * (dxv[kb][e] - xd[e] * dot[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    rs1[e] = sum16(rs1[e]);
    rs2[e] = sum16(rs2[e]);
    rowacc[e] = sum16(rowacc[e]);
    dbacc[e] = sum16(dbacc[e]);
  }
  float Fsum_part = 0.f;
  if (!hi) {
    if (col == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * wr + 4 * grp + e;
        rowq[r] = a.scale * eg[r] * rs1[e] + rowacc[e];
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * wr + 4 * grp + e;
      rs2[e] = (r < Cc) ? rs2[e] * dl[r] : 0.f;  // F_r
      Fsum_part += rs2[e];
    }
    if (col == 0) {
      fsum[wr][grp] = Fsum_part;
      // the row terms of this side for the dgamma / dbeta rows below
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * wr + 4 * grp + e;
        rowv[r] = rowacc[e];
        rowv[64 + r] = rs1[e];
        rowv[128 + r] = rs2[e];
        rowv[192 + r] = dbacc[e];
      }
    }
  }
  __syncthreads();  // every wave is done with dPG and DMs; rowq and fsum are in
  // dq (side 0) / dk (side 1) rows, once the group sum is whole: staged
  // row-major in the free S / dSn tiles for 16-byte stores
  if (store_dqk) {
    T* stage = hi ? Gs_ : Ss;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        stage[(16 * wr + 4 * grp + e) * LD + 16 * kb + col] = from_f<T>(dxv[kb][e]);
  }

  // dgamma and dbeta rows, row l on lane l of wave 4: every read of a row
  // issues at once (four rows per lane on a quarter of the lanes would chain
  // their LDS round trips)
  if (w == 4) {
    const int r = l;
    float Fs = 0.f;
    for (int ww = 0; ww < 4; ++ww)
      for (int gg = 0; gg < 4; ++gg) Fs += fsum[ww][gg];
    const float ss = ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
    float dgv = rowq[r] + rowv[r] + bex[r] * rowv[64 + r] - rowv[128 + r];
    if (r == Cc - 1) dgv += Fs + __expf(gam[63]) * ss;
    dgam[r] += dgv;
    const float db = dbv[0][r] + dbv[1][r] + dbv[2][r] + dbv[3][r] + dbv[4][r] + dbv[5][r] +
                     dbv[6][r] + dbv[7][r] + eg[r] * rowv[64 + r] + rowv[192 + r];
    if (r < Cc) reinterpret_cast<T*>(a.dbeta)[(t0 + r) * a.Hv + h] = from_f<T>(db * dbf[r]);
  }
  __syncthreads();
  if (store_dqk) {
    tile_from_lds<T, 128, 512, true>(reinterpret_cast<T*>(a.dq) + (t0 * a.Hq + hq) * kDim,
                               (int64_t)a.Hq * kDim, Ss, LD, Cc);
    tile_from_lds<T, 128, 512, true>(reinterpret_cast<T*>(a.dk) + (t0 * a.Hq + hq) * kDim,
                               (int64_t)a.Hq * kDim, Gs_, LD, Cc);
  }
  // dg = reverse cumsum of dgamma over the valid rows: lane l scans row 63 - l
  if (w == 0) {
    const int r = 63 - l;
    float x = wave_inclusive_scan(r < Cc ? dgam[r] : 0.f);
    if (a.gate_A_log) {
      // x is the gradient of the row's log decay; the gate input's gradient is
      // x times the gate's slope, and the chunk's shares of d A_log and
      // d dt_bias are the sums of x * logdecay and of that gradient (rows
      // past the chunk's end hold zero slope and log decay)
      const float pa = x * gsl[1][r];
      x *= gsl[0][r];
      const float sa = sum4g(sum16(pa)), sb = sum4g(sum16(x));
      if (l == 0) {
        a.gpart[((int64_t)c * a.Hv + h) * 2] = sa;
        a.gpart[((int64_t)c * a.Hv + h) * 2 + 1] = sb;
      }
    }
    if (r < Cc) store_scalar(a.dg, (t0 + r) * a.Hv + h, a.g_dtype, x);
  }
}

template <typename T, bool QKN, bool GVA>
__global__ __launch_bounds__(512) void grad_kernel(GradArgs a) {
  __shared__ GradLds<T> lds;
  GradFirst<T> f;
  grad_body<T, QKN, GVA>(a, (int)blockIdx.x, (int)blockIdx.y, (int)gridDim.x, lds, f);
}

// The gradient pass over ngx chunk rows x rows workgroup rows, one
// workgroup per item.
template <typename T, bool GVA>
static void launch_grad(const GradArgs& ga, int ngx, int rows, hipStream_t st) {
  if (ngx <= 0 || rows <= 0) return;
  if (ga.qk_norm)
    GDR_LAUNCH("grad", (grad_kernel<T, true, GVA>), dim3(ngx, rows), dim3(512), st, ga);
  else
    GDR_LAUNCH("grad", (grad_kernel<T, false, GVA>), dim3(ngx, rows), dim3(512), st, ga);
}

// Pipelined backward (dense batches, one segment per sequence): the
// state-gradient scan runs in slices of chunks, last slice first, and each
// launch after the first also runs the gradient workgroups of the slice the
// launch before finished.  Blocks [0, nb2) take the scan slice (one 64-column
// block each, dispatched first, so they start on free CUs); the rest take
// gradient workgroups, ngx chunk rows per head, on the CUs the scan leaves
// idle and then on all of them.  The kernel boundary between launches orders
// a slice's state gradients before their gradient workgroups read them.
template <typename T, int OPT>
__global__ __launch_bounds__(512) void bwd_pipe_kernel(DhArgs da, GradArgs ga, int nb2, int ngx) {
  typedef typename std::conditional<(OPT & 1) != 0, DhLhLds<T>, DhLdLds<T>>::type L2;
  constexpr size_t B = sizeof(L2), G = sizeof(GradLds<T>);
  __shared__ __align__(16) char lds[B > G ? B : G];
  if ((int)blockIdx.x < nb2) {
    if constexpr ((OPT & 1) != 0)
      dh_lh_body<T, OPT>(da, (int)blockIdx.x, nb2, *reinterpret_cast<L2*>(lds));
    else
      dh_ld_body<T, OPT>(da, (int)blockIdx.x, nb2, *reinterpret_cast<L2*>(lds));
  } else {
    const int g = (int)blockIdx.x - nb2;
    GradFirst<T> f;
    grad_body<T, (OPT & 1) != 0, false>(ga, g % ngx, g / ngx, ngx,
                                        *reinterpret_cast<GradLds<T>*>(lds), f);
  }
}

// The backward of a batch with few (sequence, head) units in one launch,
// scheduled by data: blocks [0, nb2) run the state-gradient scan over every
// chunk (loader-wave form, one 128-column workgroup per unit), the rest are
// the gradient workgroups, the last chunk's first (dense: row g is chunk
// nch - 1 - g / rows of workgroup row g % rows, rows per chunk; with GVA the
// rows of value heads 0 .. G-2 of every group, whose group sums the gradient
// kernel completes in a launch of its own; packed sequences: item g / Hv of
// the item table, head g % Hv).  Blocks are dispatched in order, so the
// scan's workgroups are resident before any gradient workgroup waits for
// them; a gradient workgroup waits (bounded) until its unit's count covers
// its chunk's state gradient, then runs on whatever CU it was given: the
// chip's idle CUs during the scan, every CU after it.
constexpr int kDynSpinLimit = 1 << 20;  // about 0.25 s of s_sleep: never reached in a healthy run
// OPT bit 0: q and k hold rows normalised beforehand (GradArgs::qinv), which
// the scan reads as they are and the gradient workgroups map dq, dk back
// through; bit 1: the beta options.
template <typename T, int OPT, bool GVA>
__global__ __launch_bounds__(512) void bwd_dyn_kernel(DhArgs da, GradArgs ga, int nb2) {
  constexpr size_t B = sizeof(DhLdLds<T, 2>), G = sizeof(GradLds<T>);
  __shared__ __align__(16) char lds[B > G ? B : G];
  if ((int)blockIdx.x < nb2) {
    dh_ld_body<T, OPT & 2, 2, (GVA ? 1 : 0) | (OPT & 1 ? 2 : 0)>(
        da, (int)blockIdx.x, nb2, *reinterpret_cast<DhLdLds<T, 2>*>(lds));
    return;
  }
  const int g = (int)blockIdx.x - nb2, units = ga.N * ga.Hv, nch = ga.nc_dense;
  int j, n, by, u, nc = nch;
  if (!GVA && ga.items) {  // packed sequences: the item table's order
    n = ga.items[2 * (g / ga.Hv)];
    j = ga.items[2 * (g / ga.Hv) + 1];
    by = g % ga.Hv;
    u = n * ga.Hv + by;
    nc = ga.offs[n + 1] - ga.offs[n];
  } else if constexpr (GVA) {
    const int gs = ga.Hv / ga.Hq, hrow = ga.Hq * (gs - 1);  // workgroup rows per (sequence, chunk)
    const int rows = ga.N * hrow, x = g % rows;
    j = nch - 1 - g / rows;
    n = x / hrow;
    by = x % hrow;
    u = n * ga.Hv + (by / (gs - 1)) * gs + by % (gs - 1);
  } else {
    j = nch - 1 - g / units;
    u = g % units;
    n = u / ga.Hv;
    by = u % ga.Hv;
  }
  // every tile but the state gradient is an input of the launch: the loads
  // are issued before the wait, so their latency overlaps it
  GradFirst<T> f;
  const int c = ga.items ? ga.offs[n] + j : n * nch + j;  // global chunk row
  const GradItem item = grad_item<GVA>(ga, c, by);
  grad_first_loads<T>(ga, item, f, false);
  if (threadIdx.x == 0) {
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(ga.flags, (int64_t)units * 4);
    const unsigned need = (unsigned)(nc - j);
    for (int it = 0; it < kDynSpinLimit; ++it) {
      if (buf_load_u32_sc1(rs, u * 4) >= need) break;
      __builtin_amdgcn_s_sleep(8);
    }
  }
  // the workgroup barrier without __syncthreads' fence, which would wait for
  // the loads just issued; the acquire fence keeps the state gradient's loads
  // below it
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  grad_dsn_load<T>(ga, item, 0, f.rg);
  grad_body<T, (OPT & 1) != 0, GVA, true>(ga, c, by, ga.N * nch,
                                          *reinterpret_cast<GradLds<T>*>(lds), f);
}

// The data-scheduled backward's gradient items for packed sequences, in
// launch order: by distance from the sequence's end (the order the scan
// stores the state gradients in), within one distance the longest sequences
// first.  Sequences longer than d chunks are ranks 0 .. cnt[d]-1 of order
// (longest first), so item (sequence order[r], its chunk L-1-d) takes slot
// base[d] + r, base the exclusive prefix sum of cnt.  Also zeroes the
// progress counts.  One workgroup; maxc (the longest sequence's chunks) at
// most kDynMaxChunks.
constexpr int kDynMaxChunks = 4096;
static __global__ __launch_bounds__(256) void dyn_items_kernel(const int32_t* offs,
                                                               const int32_t* order, int N,
                                                               int maxc, int32_t* items,
                                                               int64_t nitems, unsigned* flags,
                                                               int nflags) {
  __shared__ int32_t base[kDynMaxChunks];
  __shared__ int32_t part[256];
  const int tid = (int)threadIdx.x;
  for (int i = tid; i < nflags; i += 256) flags[i] = 0u;
  for (int d = tid; d < maxc; d += 256) {  // cnt[d]: the first rank of at most d chunks
    int lo = 0, hi = N;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1, m = order[mid];
      if (offs[m + 1] - offs[m] > d) lo = mid + 1;
      else hi = mid;
    }
    base[d] = lo;
  }
  __syncthreads();
  const int per = (maxc + 255) / 256, d0 = min(maxc, tid * per), d1 = min(maxc, d0 + per);
  int sum = 0;
  for (int d = d0; d < d1; ++d) sum += base[d];
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int t = part[i];
      part[i] = acc;
      acc += t;
    }
  }
  __syncthreads();
  int acc = part[tid];
  for (int d = d0; d < d1; ++d) {
    const int t = base[d];
    base[d] = acc;
    acc += t;
  }
  __syncthreads();
  // (the host's lengths bound every slot: a device cu_seqlens that disagrees
  // with them cannot write past the table)
  for (int r = tid; r < N; r += 256) {
    const int n = order[r], L = min(offs[n + 1] - offs[n], maxc);
    for (int d = 0; d < L; ++d) {
      const int64_t slot = (int64_t)base[d] + r;
      if (slot < nitems) {
        items[2 * slot] = n;
        items[2 * slot + 1] = L - 1 - d;
      }
    }
  }
}

static __global__ void zero_u32_kernel(unsigned* p, int n) {
  for (int i = (int)threadIdx.x; i < n; i += (int)blockDim.x) p[i] = 0u;
}

// d A_log[h] and d dt_bias[h]: the per-chunk shares summed over every chunk of
// every sequence.  One workgroup per head; thread t adds chunks t, t + 256,
// ... in order, then a fixed pairwise tree combines the 256 partial sums.
__global__ __launch_bounds__(256) void gate_param_grad_kernel(const float* gpart, int64_t nchunks,
                                                              int Hv, float* dA_log,
                                                              float* ddt_bias) {
  __shared__ float ra[256], rb[256];
  const int h = blockIdx.x, t = threadIdx.x;
  float sa = 0.f, sb = 0.f;
  for (int64_t c = t; c < nchunks; c += 256) {
    sa += gpart[(c * Hv + h) * 2];
    sb += gpart[(c * Hv + h) * 2 + 1];
  }
  ra[t] = sa;
  rb[t] = sb;
  __syncthreads();
  for (int half = 128; half > 0; half >>= 1) {
    if (t < half) {
      ra[t] += ra[t + half];
      rb[t] += rb[t + half];
    }
    __syncthreads();
  }
  if (t == 0) {
    if (dA_log) dA_log[h] = ra[0];
    if (ddt_bias) ddt_bias[h] = rb[0];
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Slices of the pipelined backward (bwd_pipe_kernel), 0 when it does not
// apply: the forward's states given, a dense batch, no split along T, the
// one-tile scan, at least 16 chunks per sequence, and few enough (sequence,
// head) units that the scan leaves at least half the CUs idle: at most 128
// units for the data-scheduled launch (one 128-column workgroup each), at
// most 64 and no grouped heads for the slices (two 64-column workgroups
// each).
// 0: no pipeline; 1: one launch scheduled by data (bwd_dyn_kernel); S >= 2:
// S slices (q / k normalised in the kernel, whose scan form has no progress
// counts).
static int pipe_slices(const gdr_problem* p, const Plan& pl, bool states_given) {
  if (!states_given || pl.cp != 1 || pl.vb != 1) return 0;
  if (p->cu_seqlens_dev) {
    // packed sequences (no grouped heads): the data-scheduled launch for up
    // to 256 units, the scan's workgroups of short sequences handing their
    // CUs to the gradient workgroups as they finish
    const int64_t maxc = (pl.max_len + kChunk - 1) / kChunk;
    if (p->Hq != p->Hv || p->use_qk_l2norm || (int64_t)pl.N * p->Hv > 256 || maxc < 16 ||
        maxc > kDynMaxChunks)
      return 0;
    return 1;
  }
  if (pl.nc_dense < 16 || (int64_t)pl.N * p->Hv > 128) return 0;
  if (!p->use_qk_l2norm) return 1;
  if (p->Hq != p->Hv || (int64_t)pl.N * p->Hv * 2 > 128) return 0;
  return 2;  // measured at B=2 T=4096 H=32: 2 slices 449 us, 3 slices 455, 4 slices 498,
             // one pass 489
}

// Slice boundaries (chunks [lo[p], lo[p + 1]) form slice p; the scan walks
// slice S-1 first).  A launch runs one slice of the scan beside the gradient
// workgroups of the slice after it, so each slice is sized for those to fit
// on the CUs the scan leaves idle: r = (gradient work of one chunk index) /
// (idle CUs x scan time of one chunk), about 19 us per gradient workgroup and
// 2.9 us per scan chunk, and slice p is r times slice p + 1.
static void pipe_bounds(const gdr_problem* p, const Plan& pl, int S, int* lo) {
  if (S == 1) {  // one launch over every chunk (packed: the longest sequence's)
    lo[0] = 0;
    lo[1] = p->cu_seqlens_dev ? (int)((pl.max_len + kChunk - 1) / kChunk) : pl.nc_dense;
    return;
  }
  const double units = (double)pl.N * p->Hv;
  const double r = units * 19.0 / ((256.0 - 2.0 * units) * 2.9);
  double w[8], sum = 0.0, x = 1.0;
  for (int q = S - 1; q >= 0; --q, x *= r) sum += (w[q] = x);
  const int nch = pl.nc_dense;
  lo[S] = nch;
  for (int q = S - 1; q >= 1; --q) {
    int m = (int)(w[q] / sum * nch + 0.5);
    if (m < 1) m = 1;
    lo[q] = lo[q + 1] - m;
    if (lo[q] < q) lo[q] = q;  // every slice keeps at least one chunk
  }
  // the last launch runs slice 0's gradients alone on the whole chip: a
  // whole number of rounds of 256 workgroups where the sizes allow it
  int gq = 256;
  for (int u = (int)units; gq > 1 && u % 2 == 0; u /= 2) gq /= 2;  // 256 / gcd(256, units)
  if (gq <= lo[1] / 2 && lo[1] - lo[1] % gq >= 1) lo[1] -= lo[1] % gq;
  lo[0] = 0;
}

struct BwdLayout {
  size_t offs, cp, cp2, h, dh, gacc, gpart, pipe, flags, items, total;
};

static BwdLayout bwd_layout(const gdr_problem* p, const Plan& pl, bool states_given) {
  BwdLayout L;
  size_t o = 0;
  L.offs = o;  // chunk offsets, then the sequences' length order
  if (p->cu_seqlens_dev)
    o += align256(sizeof(int32_t) * (size_t)(pl.N + 1)) + align256(sizeof(int32_t) * (size_t)pl.N);
  // the two scans run in one launch: each has its own CP buffers
  L.cp = o;
  o += cp_workspace_bytes(pl, p->Hv);
  L.cp2 = o;
  o += cp_workspace_bytes(pl, p->Hv);
  const size_t st = (size_t)pl.total_chunks * p->Hv * kDim * kDim * 2;  // bf16/fp16
  L.h = o;
  if (!states_given) o += align256(st);
  L.dh = o;
  o += align256(st);
  L.gacc = o;
  if (p->Hq != p->Hv)
    o += align256((size_t)(p->Hv / p->Hq - 1) * pl.total_chunks * p->Hq * 8 * 8 * 64 * 4 *
                  sizeof(float));
  L.gpart = o;
  if (p->use_gate) o += align256((size_t)pl.total_chunks * p->Hv * 2 * sizeof(float));
  L.pipe = o;  // the pipelined scan's gradients between slices
  const int S = pipe_slices(p, pl, states_given);
  if (S >= 2) o += align256((size_t)pl.N * p->Hv * S * kDim * kDim * sizeof(float));
  L.flags = o;  // the data-scheduled launch's progress counts, one per unit
  if (S == 1) o += align256((size_t)pl.N * p->Hv * sizeof(unsigned));
  L.items = o;  // and its item table (packed sequences)
  if (S == 1 && p->cu_seqlens_dev) o += align256((size_t)pl.total_chunks * 2 * sizeof(int32_t));
  L.total = o;
  return L;
}

size_t bwd_workspace_bytes(const gdr_problem* p, const Plan& pl, bool states_given) {
  return bwd_layout(p, pl, states_given).total;
}

int bwd_pipe_bounds(const gdr_problem* p, const Plan& pl, bool states_given, int* lo) {
  const int S = pipe_slices(p, pl, states_given);
  if (S > 0) pipe_bounds(p, pl, S, lo);
  return S;
}

// B1 and B2 together: with CP, both augmented passes in one launch, the two
// chains (forward for B1, reverse for B2), then both output passes in one
// launch.
// With the forward's chunk states given (states_given), only the
// state-gradient scan runs: the launches keep their layout with no blocks for
// the state scan.
// With the forward's segment transitions given as well (trans), the
// state-gradient pass 1 runs only its value columns and pass 2 applies the
// forward's transitions transposed.
template <typename T, int VB>
static void launch_bwd_scans(const Plan& pl, ScanArgs sa, DhArgs da, bool states_given,
                             const float* trans, hipStream_t st) {
  const unsigned units = (unsigned)(pl.N * sa.Hv);
  if (pl.cp > 1) {
    ScanArgs s1 = sa;
    DhArgs d1 = da;
    s1.P = d1.P = pl.cp;
    s1.nvs = 4 / VB;
    d1.nvs = trans ? 2 / VB : 4 / VB;
    d1.v_only = trans ? 1 : 0;
    const unsigned n2 = units * pl.cp * d1.nvs;
    const unsigned n1 = states_given ? 0u : units * pl.cp * s1.nvs;
    if (states_given && trans && VB == 2 && !sa.qk_norm) {
      if (sa.beta_mode)
        GDR_LAUNCH("bwd_scan_aug", (dh_ld2_kernel<T, 6>), dim3(n2), dim3(512), st, d1);
      else
        GDR_LAUNCH("bwd_scan_aug", (dh_ld2_kernel<T, 4>), dim3(n2), dim3(512), st, d1);
    } else if (states_given)
      GDR_LAUNCH("bwd_scan_aug", (dh_aug_kernel<T, VB>), dim3(n2), dim3(256), st, d1);
    else
      GDR_LAUNCH("bwd_scan_aug", (bwd_scans_kernel<T, VB, MODE_AUG, MODE_AUG>), dim3(n1 + n2),
                 dim3(256), st, s1, d1, (int)n1);
    if (!states_given)
      GDR_LAUNCH("cp_combine_bwd", cp_combine_kernel, dim3(units * 8), dim3(256), st, s1);
    ScanArgs r;
    memset(&r, 0, sizeof(r));
    r.cu = da.cu;
    r.T = da.T;
    r.Hv = da.Hv;
    r.P = pl.cp;
    r.seg_out = da.seg_out;
    r.seg_start = da.seg_start;
    r.trans = const_cast<float*>(trans);
    r.reverse = 1;
    GDR_LAUNCH("cp_combine_bwd", cp_combine_kernel, dim3(units * 8), dim3(256), st, r);
  }
  sa.P = da.P = pl.cp;
  sa.nvs = da.nvs = 2 / VB;
  const unsigned n2 = units * pl.cp * sa.nvs;
  const unsigned n1 = states_given ? 0u : n2;
  const dim3 grid(n1 + n2);
  if (VB == 1 && n1 == 0 && !sa.qk_norm) {
    if (sa.beta_mode) GDR_LAUNCH("bwd_scans", (dh_ld_kernel<T, 2>), grid, dim3(512), st, da);
    else GDR_LAUNCH("bwd_scans", (dh_ld_kernel<T, 0>), grid, dim3(512), st, da);
  } else if (VB == 2 && n1 == 0 && !sa.qk_norm) {
    if (sa.beta_mode) GDR_LAUNCH("bwd_scans", (dh_ld2_kernel<T, 2>), grid, dim3(512), st, da);
    else GDR_LAUNCH("bwd_scans", (dh_ld2_kernel<T, 0>), grid, dim3(512), st, da);
  } else if (VB == 1)
    switch ((sa.qk_norm ? 1 : 0) | (sa.beta_mode ? 2 : 0)) {
      case 0:
        GDR_LAUNCH("bwd_scans", (bwd_scans_lh_kernel<T, 0>), grid, dim3(512), st, sa, da, (int)n1);
        break;
      case 1:
        GDR_LAUNCH("bwd_scans", (bwd_scans_lh_kernel<T, 1>), grid, dim3(512), st, sa, da, (int)n1);
        break;
      case 2:
        GDR_LAUNCH("bwd_scans", (bwd_scans_lh_kernel<T, 2>), grid, dim3(512), st, sa, da, (int)n1);
        break;
      default:
        GDR_LAUNCH("bwd_scans", (bwd_scans_lh_kernel<T, 3>), grid, dim3(512), st, sa, da, (int)n1);
    }
  else
    GDR_LAUNCH("bwd_scans", (bwd_scans_kernel<T, VB, MODE_STATE, MODE_OUT>), grid, dim3(256), st,
               sa, da, (int)n1);
}

template <typename T>
static gdr_status launch_bwd_t(const gdr_problem* p, const Plan& pl, const void* q, const void* k,
                               const void* v, const float* gcum, const void* graw,
                               const void* beta, const void* A, const void* dO, const float* dht,
                               const float* h0, const void* hstates, const float* trans,
                               void* dq, void* dk, void* dv, void* dbeta, void* dg, float* dh0,
                               float* dA_log, float* ddt_bias, char* ws, hipStream_t st,
                               const float* qinv, const float* kinv) {
  const bool states_given = hstates != nullptr;
  const BwdLayout L = bwd_layout(p, pl, states_given);
  const int32_t* offs = nullptr;
  const int32_t* order = nullptr;
  if (p->cu_seqlens_dev) {
    int32_t* o32 = reinterpret_cast<int32_t*>(ws + L.offs);
    int32_t* r32 = reinterpret_cast<int32_t*>(ws + L.offs +
                                              align256(sizeof(int32_t) * (size_t)(pl.N + 1)));
    GDR_LAUNCH("chunk_offsets", chunk_offsets_kernel, dim3(1), dim3(256), st, p->cu_seqlens_dev,
               pl.N, o32, r32);
    offs = o32;
    order = r32;
  }
  float* cp_out = nullptr;
  float* cp_start = nullptr;
  float* cp2_out = nullptr;
  float* cp2_start = nullptr;
  if (pl.cp > 1) {
    const size_t units = (size_t)pl.N * p->Hv;
    const size_t so = align256(units * pl.cp * 2 * kDim * kDim * sizeof(float));
    cp_out = reinterpret_cast<float*>(ws + L.cp);
    cp_start = reinterpret_cast<float*>(ws + L.cp + so);
    cp2_out = reinterpret_cast<float*>(ws + L.cp2);
    cp2_start = reinterpret_cast<float*>(ws + L.cp2 + so);
  }
  void* hbuf = states_given ? const_cast<void*>(hstates) : (void*)(ws + L.h);
  void* dhbuf = ws + L.dh;
  // B1: chunk-start states (packed)
  ScanArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.q = q; sa.k = k; sa.v = v; sa.beta = beta; sa.gcum = gcum; sa.A = A; sa.h0 = h0;
  sa.h = hbuf;
  sa.cu = p->cu_seqlens_dev; sa.offs = offs; sa.order = order;
  sa.N = pl.N; sa.T = p->T; sa.Hq = p->Hq; sa.Hv = p->Hv; sa.nc_dense = pl.nc_dense;
  sa.P = 1; sa.nvs = 1; sa.scale = p->scale; sa.svf = p->state_v_first ? 1 : 0; sa.h_svf = 1;
  sa.qk_norm = p->use_qk_l2norm ? 1 : 0;
  sa.beta_mode = (p->beta_sigmoid ? 1 : 0) | (p->neg_eigval ? 2 : 0);
  sa.seg_out = cp_out; sa.seg_start = cp_start; sa.reverse = 0;
  // B2: state gradients (packed)
  DhArgs da;
  memset(&da, 0, sizeof(da));
  da.q = q; da.k = k; da.dO = dO; da.beta = beta; da.gcum = gcum; da.A = A; da.dht = dht;
  da.dh = dhbuf; da.dh0 = dh0; da.seg_start = cp2_start; da.seg_out = cp2_out;
  da.cu = p->cu_seqlens_dev; da.offs = offs; da.order = order;
  da.N = pl.N; da.T = p->T; da.Hq = p->Hq; da.Hv = p->Hv; da.nc_dense = pl.nc_dense;
  da.P = 1; da.nvs = 1; da.scale = p->scale; da.svf = sa.svf; da.qk_norm = sa.qk_norm;
  da.beta_mode = sa.beta_mode;
  const int S = pipe_slices(p, pl, states_given);
  if (S == 0) {
    if (pl.vb == 2) launch_bwd_scans<T, 2>(pl, sa, da, states_given, trans, st);
    else launch_bwd_scans<T, 1>(pl, sa, da, states_given, trans, st);
  }
  // B3-B6
  const bool gva = p->Hq != p->Hv;
  GradArgs ga;
  memset(&ga, 0, sizeof(ga));
  ga.q = q; ga.k = k; ga.v = v; ga.dO = dO; ga.beta = beta; ga.gcum = gcum; ga.A = A;
  ga.h = hbuf; ga.dh = dhbuf;
  ga.dq = dq;
  ga.dk = dk;
  ga.gacc = gva ? reinterpret_cast<float*>(ws + L.gacc) : nullptr;
  ga.dv = dv; ga.dbeta = dbeta; ga.dg = dg;
  ga.cu = p->cu_seqlens_dev; ga.offs = offs;
  ga.N = pl.N; ga.T = p->T; ga.Hq = p->Hq; ga.Hv = p->Hv; ga.nc_dense = pl.nc_dense;
  ga.g_dtype = (int)p->g_dtype; ga.scale = p->scale;
  ga.qk_norm = sa.qk_norm || qinv ? 1 : 0;  // unit rows given: the map of dq, dk only
  ga.qinv = qinv;
  ga.kinv = kinv;
  ga.beta_mode = sa.beta_mode;
  const bool gate = p->use_gate != 0;
  ga.graw = gate ? graw : nullptr;
  ga.gate_A_log = gate ? p->gate_A_log : nullptr;
  ga.gate_dt_bias = gate ? p->gate_dt_bias : nullptr;
  ga.gpart = gate ? reinterpret_cast<float*>(ws + L.gpart) : nullptr;
  // one workgroup per (chunk, value head); with GVA the heads 0 .. G-2 of
  // every group first, then the group's last head, which sums dq and dk
  const unsigned nc = (unsigned)pl.total_chunks;
  const int G = p->Hv / p->Hq;
  ga.gva_final = 0;
  if (S == 1) {
    // one launch: the scan's units workgroups (128 columns each), then the gradient
    // workgroups of every chunk, last chunk first, each waiting for its
    // chunk's state gradient (progress counts zeroed by a kernel, so that a
    // captured graph replays correctly)
    const int units = pl.N * p->Hv, nb2 = units;
    unsigned* flags = reinterpret_cast<unsigned*>(ws + L.flags);
    int32_t* items = nullptr;
    if (p->cu_seqlens_dev) {
      items = reinterpret_cast<int32_t*>(ws + L.items);
      GDR_LAUNCH("bwd_flags", dyn_items_kernel, dim3(1), dim3(256), st, offs, order, pl.N,
                 (int)((pl.max_len + kChunk - 1) / kChunk), items, (int64_t)pl.total_chunks,
                 flags, units);
    } else {
      GDR_LAUNCH("bwd_flags", zero_u32_kernel, dim3(1), dim3(256), st, flags, units);
    }
    DhArgs d = da;
    d.P = 1;
    d.nvs = 1;
    d.flags = flags;
    GradArgs g2 = ga;
    g2.flags = flags;
    g2.items = items;
    // with GVA the launch takes value heads 0 .. G-2 of every group; the
    // gradient kernel then runs the group's last head, which sums dq and dk
    const int rows = gva ? pl.N * p->Hq * (G - 1) : units;
    const unsigned blocks = (unsigned)(items ? nb2 + pl.total_chunks * p->Hv
                                             : nb2 + (int64_t)rows * pl.nc_dense);
    switch ((qinv ? 4 : 0) | (sa.beta_mode ? 2 : 0) | (gva ? 1 : 0)) {
      case 0: GDR_LAUNCH("bwd_dyn", (bwd_dyn_kernel<T, 0, false>), dim3(blocks), dim3(512), st, d, g2, nb2); break;
      case 1: GDR_LAUNCH("bwd_dyn", (bwd_dyn_kernel<T, 0, true>), dim3(blocks), dim3(512), st, d, g2, nb2); break;
      case 2: GDR_LAUNCH("bwd_dyn", (bwd_dyn_kernel<T, 2, false>), dim3(blocks), dim3(512), st, d, g2, nb2); break;
      case 3: GDR_LAUNCH("bwd_dyn", (bwd_dyn_kernel<T, 2, true>), dim3(blocks), dim3(512), st, d, g2, nb2); break;
      case 4: GDR_LAUNCH("bwd_dyn", (bwd_dyn_kernel<T, 1, false>), dim3(blocks), dim3(512), st, d, g2, nb2); break;
      case 5: GDR_LAUNCH("bwd_dyn", (bwd_dyn_kernel<T, 1, true>), dim3(blocks), dim3(512), st, d, g2, nb2); break;
      case 6: GDR_LAUNCH("bwd_dyn", (bwd_dyn_kernel<T, 3, false>), dim3(blocks), dim3(512), st, d, g2, nb2); break;
      default: GDR_LAUNCH("bwd_dyn", (bwd_dyn_kernel<T, 3, true>), dim3(blocks), dim3(512), st, d, g2, nb2);
    }
    if (gva) {
      ga.gva_final = 1;
      launch_grad<T, true>(ga, (int)nc, p->Hq, st);
    }
  } else if (S > 0) {
    // launch k runs scan slice S-1-k (while k < S) and the gradient
    // workgroups of slice S-k (once k > 0)
    DhArgs d = da;
    d.P = S;
    d.nvs = 2;
    d.sliced = 1;
    d.seg_start = d.seg_next = reinterpret_cast<float*>(ws + L.pipe);
    const int nb2 = pl.N * p->Hv * 2;
    int lo[9];
    bwd_pipe_bounds(p, pl, states_given, lo);
    const int opt = (sa.qk_norm ? 1 : 0) | (sa.beta_mode ? 2 : 0);
    for (int k = 0; k <= S; ++k) {
      const int pb = S - 1 - k, pg = S - k;
      GradArgs g2 = ga;
      int ngx = 0;
      if (pg < S) {
        g2.sl_c0 = lo[pg];
        g2.sl_len = lo[pg + 1] - lo[pg];
        ngx = pl.N * g2.sl_len;
      }
      d.slice_p = pb >= 0 ? pb : 0;
      d.sl_c0 = pb >= 0 ? lo[pb] : 0;
      d.sl_c1 = pb >= 0 ? lo[pb + 1] : 0;
      const int b2 = pb >= 0 ? nb2 : 0;
      const unsigned blocks = (unsigned)(b2 + ngx * p->Hv);
      if (blocks == 0) continue;
      if (b2 == 0) {  // the last slice's gradients alone: the gradient kernel itself
        launch_grad<T, false>(g2, ngx, p->Hv, st);
        continue;
      }
      switch (opt) {
        case 0: GDR_LAUNCH("bwd_pipe", (bwd_pipe_kernel<T, 0>), dim3(blocks), dim3(512), st, d, g2, b2, ngx); break;
        case 1: GDR_LAUNCH("bwd_pipe", (bwd_pipe_kernel<T, 1>), dim3(blocks), dim3(512), st, d, g2, b2, ngx); break;
        case 2: GDR_LAUNCH("bwd_pipe", (bwd_pipe_kernel<T, 2>), dim3(blocks), dim3(512), st, d, g2, b2, ngx); break;
        default: GDR_LAUNCH("bwd_pipe", (bwd_pipe_kernel<T, 3>), dim3(blocks), dim3(512), st, d, g2, b2, ngx);
      }
    }
  } else if (pl.total_chunks > 0 && !gva) {
    launch_grad<T, false>(ga, (int)nc, p->Hv, st);
  } else if (pl.total_chunks > 0) {
    for (int fin = 0; fin < 2; ++fin) {
      ga.gva_final = fin;
      launch_grad<T, true>(ga, (int)nc, fin ? p->Hq : p->Hq * (G - 1), st);
    }
  }
  if (gate && (dA_log || ddt_bias))
    GDR_LAUNCH("gate_param_grad", gate_param_grad_kernel, dim3((unsigned)p->Hv), dim3(256), st,
               ga.gpart, (int64_t)pl.total_chunks, p->Hv, dA_log, ddt_bias);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("backward launch failed: %s", hipGetErrorString(e));
    return GDR_ERR_HIP;
  }
  return GDR_OK;
}

gdr_status launch_bwd(const gdr_problem* p, const Plan& pl, const void* q, const void* k,
                      const void* v, const float* gcum, const void* graw, const void* beta,
                      const void* A, const void* dO, const float* dht, const float* h0,
                      const void* hstates, const float* trans, void* dq, void* dk, void* dv,
                      void* dbeta, void* dg, float* dh0, float* dA_log, float* ddt_bias, void* ws,
                      hipStream_t st, const float* qinv, const float* kinv) {
  char* w = reinterpret_cast<char*>(ws);
  if (trans && !hstates) {
    set_error("segment transitions come with the forward's states");
    return GDR_ERR_ARG;
  }
  if ((qinv != nullptr) != (kinv != nullptr) || (qinv && p->use_qk_l2norm)) {
    set_error("normalised rows come with both norms, on a problem that does not normalise");
    return GDR_ERR_ARG;
  }
  if (p->in_dtype == GDR_BF16)
    return launch_bwd_t<__bf16>(p, pl, q, k, v, gcum, graw, beta, A, dO, dht, h0, hstates, trans,
                                dq, dk, dv, dbeta, dg, dh0, dA_log, ddt_bias, w, st, qinv, kinv);
  return launch_bwd_t<_Float16>(p, pl, q, k, v, gcum, graw, beta, A, dO, dht, h0, hstates, trans,
                                dq, dk, dv, dbeta, dg, dh0, dA_log, ddt_bias, w, st, qinv, kinv);
}

}  // namespace gdr

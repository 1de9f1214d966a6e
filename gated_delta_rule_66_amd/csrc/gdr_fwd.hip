// gdr_fwd.hip -- forward kernels of the chunked gated delta rule on gfx950.
//
// The forward of the FlashQLA pages ("flashqla-linear-attention", Low-Level
// API; "FlashQLA Documentation", forward pass: g, A, o, h, final_state) in two
// launches:
//
//   fwd_prep  one workgroup per (chunk, value head), fully parallel:
//             gamma = chunk-local inclusive cumsum of g            -> g_cum
//             M = strict_lower(diag(beta) K K^T o exp(gamma_r - gamma_i))
//             A = (I + M)^{-1}, unit lower triangular (fp32, blocked:
//             16x16 diagonal blocks by substitution, off-diagonal blocks by
//             fp32 MFMA)                                            -> A
//   fwd_scan  one workgroup per (sequence, value head), sequential over the
//             sequence's chunks; wave w owns value columns [32w, 32w+32) of
//             the 128 x 128 fp32 state S, held in MFMA accumulators:
//             R = diag(beta) V - diag(beta e^gamma) (K S)
//             Delta = A R                   (= U - W S of the WY form)
//             O = scale (diag(e^gamma) Q S + lower_incl(Q K^T o Gamma) Delta)
//             S <- e^{gamma_L} S + K^T (diag(e^{gamma_L - gamma}) Delta)
//
// Every contraction is a 16x16x32 bf16/fp16 MFMA with fp32 accumulation;
// S and R, Delta enter the next product as register-local B operands.
#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_scan.h"

#include <cstring>
#include <mutex>

namespace gdr {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* h0;
  float* gcum;
  void* A;
  void* o;
  void* h;
  float* ht;
  const int32_t* cu;    // device cu_seqlens, or null for dense batches
  const int32_t* offs;  // device chunk offsets [N+1] (packed input only)
  int N, T, Hq, Hv;
  int nc_dense;
  int g_dtype;
  float scale;
  int svf;
  int qk_norm;    // q, k rows scaled to unit length before use
  int beta_mode;  // bit 0 sigmoid of a beta logit, bit 1 twice beta
  const float* gate_A_log;    // non-null: g is the gate input (gate_log_decay)
  const float* gate_dt_bias;  // nullable
  // (qk_norm) non-null: the group's first value head also writes the unit q
  // and k rows of its chunk (q's layout) and their fp32 1 / |x| per (token,
  // q head), which the scans and the backward then read instead
  void* qn;
  void* kn;
  float* qinv;
  float* kinv;
};

// KEEP: a.qn is set (the states path with q / k normalised): the group's
// first value head also keeps the unit rows and their norms.
template <typename T, bool KEEP>
__device__ __forceinline__ void fwd_prep_item(const FwdArgs& a, const int c, const int h) {
  // LDS, 26 KB per workgroup (six workgroups per CU): the k tile, swizzled
  // (sw_off, 16 KB), and M.  Only the ten 16 x 16 blocks on or below the
  // diagonal of M and of the inverse are ever written or read: block
  // (bi, bj), bj <= bi, sits at slot bi (bi + 1) / 2 + bj.  The k tile is
  // dead once M is formed (a barrier follows), so the inverse's blocks
  // (rows 20 floats apart, 12.5 KB) take its storage.  M's rows are 16 floats
  // with column c of row r at (c + 4 ((r / 4) % 4)) % 16: the inverse's
  // products read 16 rows of one column group at once, and over rows
  // 0 .. 15 of a block that rotation puts them on distinct banks.
  __shared__ __align__(16) T Ks[64 * 128];
  float* const Ai = reinterpret_cast<float*>(Ks);
  __shared__ __align__(16) float Mf[10 * 16 * 16];
  auto slot = [](int r, int c) { return (r >> 4) * ((r >> 4) + 1) / 2 + (c >> 4); };
  auto ai = [&](int r, int c) { return (slot(r, c) * 16 + (r & 15)) * 20 + (c & 15); };
  auto mf = [&](int r, int c) {
    return (slot(r, c) * 16 + (r & 15)) * 16 + (((c & 15) + 4 * ((r >> 2) & 3)) & 15);
  };
  static_assert((9 * 16 + 15) * 20 + 16 <= 64 * 128 * (int)sizeof(T) / 4,
                "the inverse's blocks fit in the k tile's storage");

  int n, j;
  if (a.cu) {
    n = find_seq(a.offs, a.N, c);
    j = c - a.offs[n];
  } else {
    n = c / a.nc_dense;
    j = c % a.nc_dense;
  }
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int64_t t0 = s.start + (int64_t)kChunk * j;
  const int Cc = (int)min((int64_t)kChunk, s.end - t0);
  const int G = a.Hv / a.Hq, hq = h / G;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;

  // The row's g and beta are loaded as raw bits from a clamped row by every
  // wave, with no branch around the loads (a load inside a branch ends with
  // a wait for every load issued before it): two 16-bit loads give the bits
  // of an fp32 g, or a 16-bit g in the low half (the other half is unused,
  // or past the range and zero).  The k tile follows; g and beta are
  // converted after the tile is stored.
  const int gsz = a.g_dtype == 2 ? 4 : 2;
  const int ld_g = a.Hv * gsz, rr = min(l, Cc - 1);
  const __amdgpu_buffer_rsrc_t grs =
      buf_rsrc(reinterpret_cast<const char*>(a.g) + (t0 * a.Hv + h) * (int64_t)gsz, (int64_t)Cc * ld_g);
  const __amdgpu_buffer_rsrc_t brs =
      buf_rsrc(reinterpret_cast<const T*>(a.beta) + (t0 * a.Hv + h), (int64_t)Cc * a.Hv * (int64_t)sizeof(T));
  const uint32_t glo = __builtin_amdgcn_raw_buffer_load_b16(grs, rr * ld_g, 0, 0);
  const uint32_t ghi = __builtin_amdgcn_raw_buffer_load_b16(grs, rr * ld_g + 2, 0, 0);
  const uint16_t braw = __builtin_amdgcn_raw_buffer_load_b16(brs, rr * a.Hv * (int)sizeof(T), 0, 0);
  TileRegs<128, 256> rk, rq;
  tile_load<T, 128, 256>(rk, reinterpret_cast<const T*>(a.k) + (t0 * a.Hq + hq) * kDim,
                         (int64_t)a.Hq * kDim, Cc);
  // the unit q rows when this workgroup keeps them (a q load over no rows,
  // zeros, for the group's other heads: no branch around the load)
  const bool keep_qk = KEEP && h % G == 0;
  if (KEEP)
    tile_load<T, 128, 256>(rq, reinterpret_cast<const T*>(a.q) + (t0 * a.Hq + hq) * kDim,
                           (int64_t)a.Hq * kDim, keep_qk ? Cc : 0);
  __shared__ float rinv[2][KEEP ? 64 : 1];  // 1 / |x| of the kept rows: q, k
  if (a.qk_norm) l2norm_rows<T, 256>(rk, keep_qk ? rinv[1] : nullptr);
  if (keep_qk) {
    l2norm_rows<T, 256>(rq, rinv[0]);
    const int gs = a.Hq * kDim * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t qs =
        buf_rsrc(reinterpret_cast<T*>(a.qn) + (t0 * a.Hq + hq) * kDim, (int64_t)Cc * gs);
    const __amdgpu_buffer_rsrc_t ks =
        buf_rsrc(reinterpret_cast<T*>(a.kn) + (t0 * a.Hq + hq) * kDim, (int64_t)Cc * gs);
#pragma unroll
    for (int i = 0; i < TileRegs<128, 256>::N; ++i) {
      const int x = tid + i * 256;
      buf_store16(qs, (x >> 4) * gs + (x & 15) * 16, rq.r[i]);
      buf_store16(ks, (x >> 4) * gs + (x & 15) * 16, rk.r[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < TileRegs<128, 256>::N; ++i) {
    const int x = tid + i * 256;  // 16-byte piece x % 16 of row x / 16
    *reinterpret_cast<uint4*>(Ks + sw_off<128>(x >> 4, 8 * (x & 15))) = rk.r[i];
  }
  // every wave forms the gate cumsum itself (lane l: row l) and takes the
  // rows' values it needs by lane shuffles; wave 0 stores it
  float gv = a.g_dtype == 2 ? __builtin_bit_cast(float, glo | (ghi << 16))
             : a.g_dtype == 0 ? __builtin_bit_cast(float, glo << 16)
                              : (float)__builtin_bit_cast(_Float16, (uint16_t)glo);
  if (a.gate_A_log)
    gv = gate_log_decay(gv, a.gate_A_log[h], a.gate_dt_bias ? a.gate_dt_bias[h] : 0.f);
  if (l >= Cc) gv = 0.f;
  const float bv = (l < Cc) ? beta_used(to_f(__builtin_bit_cast(T, braw)), a.beta_mode) : 0.f;
  const float gc = wave_inclusive_scan(gv);
  if (w == 0 && l < Cc) a.gcum[(t0 + l) * a.Hv + h] = gc;
  __syncthreads();
  if (keep_qk && tid < Cc) {
    a.qinv[(t0 + tid) * a.Hq + hq] = rinv[0][tid];
    a.kinv[(t0 + tid) * a.Hq + hq] = rinv[1][tid];
  }

  // M, rows 16w .. 16w+15 (only the blocks on or below the diagonal are nonzero)
  float gr[4], br[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    gr[e] = __shfl(gc, 16 * w + 4 * grp + e);
    br[e] = __shfl(bv, 16 * w + 4 * grp + e);
  }
  for (int cb = 0; cb < 4; ++cb) {
    if (cb <= w) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma16(frag_row_w<T, 128>(Ks, 16 * w, 32 * kk),
                     frag_row_w<T, 128>(Ks, 16 * cb, 32 * kk), acc);
      const float gi = __shfl(gc, 16 * cb + col);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + 4 * grp + e, i = 16 * cb + col;
        // masked entries take exp(-inf) = 0 (an unconditional exponential)
        Mf[mf(r, i)] = br[e] * __expf(i < r ? gr[e] - gi : -INFINITY) * acc[e];
      }
    }
  }
  // (the blocks of the inverse above the diagonal are never read)
  __syncthreads();

  // diagonal 16x16 blocks: forward substitution, lane l < 16 owns column l
  if (l < 16) {
    const int b0 = 16 * w;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == l) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc -= Mf[mf(b0 + r, b0 + i)] * x[i];
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Ai[ai(b0 + r, b0 + l)] = x[r];
  }
  __syncthreads();

  // off-diagonal blocks by distance d from the diagonal:
  //   A_ij = -A_ii * sum_{j <= m < i} M_im A_mj
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int bi = w + d, bj = w;
      f32x4 t = zero4();
      for (int m = bj; m < bi; ++m) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float av = Mf[mf(16 * bi + col, 16 * m + 4 * st + grp)];
          const float bv2 = Ai[ai(16 * m + 4 * st + grp, 16 * bj + col)];
          t = mfma16f32(av, bv2, t);
        }
      }
      // t is a D tile: lane (grp, col) holds t[4 grp + e][col]; step e of the
      // next product uses k = 4 grp + e for lane group grp.
      f32x4 r = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float av = Ai[ai(16 * bi + col, 16 * bi + 4 * grp + e)];
        r = mfma16f32(av, t[e], r);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Ai[ai(16 * bi + 4 * grp + e, 16 * bj + col)] = -r[e];
    }
    __syncthreads();
  }

  // A rows of the chunk, 8 elements (16 bytes) per store
  T* Aout = reinterpret_cast<T*>(a.A);
  for (int x = tid; x < 64 * 8; x += 256) {
    const int r = x >> 3, c8 = (x & 7) * 8;
    if (r < Cc) {
      typename VT<T>::x8 vals;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cc = c8 + e;
        vals[e] = from_f<T>(cc <= r ? Ai[ai(r, cc)] : 0.f);
      }
      *reinterpret_cast<typename VT<T>::x8*>(Aout + ((t0 + r) * a.Hv + h) * kChunk + c8) = vals;
    }
  }
}


// Workgroups take (chunk row c, value head h) pairs in the order c * Hv + h,
// each XCD a contiguous range of them (xcd_block), so the heads of a chunk run
// together on one XCD: the workgroups in flight read whole token rows of k,
// g and beta and write whole rows of A and g_cum, and the g, beta and g_cum
// lines that the heads share stay in that XCD's L2.  Past 2^31 - 1 pairs the
// grid is (chunk, head).
template <typename T, bool KEEP>
__global__ __launch_bounds__(256) void fwd_prep_kernel(FwdArgs a) {
  if (gridDim.y > 1) {
    fwd_prep_item<T, KEEP>(a, (int)blockIdx.x, (int)blockIdx.y);
  } else {
    const int L = xcd_block((int)blockIdx.x, (int)gridDim.x);
    fwd_prep_item<T, KEEP>(a, L / a.Hv, L % a.Hv);
  }
}


// ---- scratch of the no-allocation forward ---------------------------------
// A file-scope device array that stands in for the caller's workspace in
// gdr_chunk_fwd_noalloc.  Each GPU the library runs on holds its own copy from
// module load until the process ends.  In host code `scratch` only names the
// symbol: its device address on the current device comes from
// hipGetSymbolAddress, resolved once per device and kept.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

gdr_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    set_error("no HIP device is available");
    return GDR_ERR_DEVICE;
  }
  if (dev >= kMaxDevices) {
    set_error("device %d is past the %d devices the scratch table tracks", dev, kMaxDevices);
    return GDR_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      set_error("hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                hipGetErrorString(e));
      (void)hipGetLastError();
      return GDR_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GDR_OK;
}

size_t cp_workspace_bytes(const Plan& pl, int Hv) {
  if (pl.cp <= 1) return 0;
  const size_t units = (size_t)pl.N * Hv;
  const size_t KV = (size_t)kDim * kDim;
  return align256(units * pl.cp * 2 * KV * sizeof(float)) +
         align256(units * pl.cp * KV * sizeof(float));
}

size_t fwd_workspace_bytes(const gdr_problem* p, const Plan& pl) {
  size_t b = 0;
  if (p->cu_seqlens_dev)  // chunk offsets and the sequences' length order
    b += align256(sizeof(int32_t) * (size_t)(pl.N + 1)) + align256(sizeof(int32_t) * (size_t)pl.N);
  b += cp_workspace_bytes(pl, p->Hv);
  return b;
}

template <typename T, int VB>
static void launch_scan_vb(const Plan& pl, ScanArgs a, int mode, hipStream_t st) {
  const unsigned units = (unsigned)(pl.N * a.Hv);
  if (pl.cp > 1) {
    ScanArgs a1 = a;
    a1.P = pl.cp;
    a1.nvs = 4 / VB;
    GDR_LAUNCH("scan_aug", (scan_kernel<T, VB, MODE_AUG>), dim3(units * pl.cp * a1.nvs), dim3(256),
               st, a1);
    GDR_LAUNCH("cp_combine_fwd", cp_combine_kernel, dim3(units * 8), dim3(256), st, a1);
  }
  a.P = pl.cp;
  a.nvs = 2 / VB;
  const dim3 grid(units * pl.cp * a.nvs);
  // With 64-column workgroups filling at most half of the 256 CUs, the
  // output pass splits the value columns in four (two state waves each), so
  // the idle CUs take half of every workgroup's output work.
  const bool narrow = units * pl.cp * 2 <= 128;
  // packed h is stored by the output waves of the wave-specialized pass from
  // the state waves' operand copies; the user layouts by the 4-wave pass
  if (mode == MODE_OUT && a.h && (VB == 2 || !a.h_vm))
    GDR_LAUNCH("scan_out", (scan_kernel<T, VB, MODE_OUT_H>), grid, dim3(256), st, a);
  else if (mode == MODE_OUT && VB == 1 && narrow) {
    a.nvs = 4;
    const dim3 g4(units * pl.cp * 4);
    switch ((a.qk_norm ? 1 : 0) | (a.beta_mode ? 2 : 0)) {
      case 0: GDR_LAUNCH("scan_out", (scan_out_ld_kernel<T, 0>), g4, dim3(512), st, a); break;
      case 1: GDR_LAUNCH("scan_out", (scan_out_kernel<T, 1, 2>), g4, dim3(384), st, a); break;
      case 2: GDR_LAUNCH("scan_out", (scan_out_ld_kernel<T, 2>), g4, dim3(512), st, a); break;
      default: GDR_LAUNCH("scan_out", (scan_out_kernel<T, 3, 2>), g4, dim3(384), st, a);
    }
  } else if (mode == MODE_OUT && VB == 1) {
    switch ((a.qk_norm ? 1 : 0) | (a.beta_mode ? 2 : 0)) {
      case 0: GDR_LAUNCH("scan_out", (scan_out_kernel<T, 0, 4>), grid, dim3(512), st, a); break;
      case 1: GDR_LAUNCH("scan_out", (scan_out_kernel<T, 1, 4>), grid, dim3(512), st, a); break;
      case 2: GDR_LAUNCH("scan_out", (scan_out_kernel<T, 2, 4>), grid, dim3(512), st, a); break;
      default: GDR_LAUNCH("scan_out", (scan_out_kernel<T, 3, 4>), grid, dim3(512), st, a);
    }
  }
  else if (mode == MODE_OUT)
    GDR_LAUNCH("scan_out", (scan_kernel<T, VB, MODE_OUT>), grid, dim3(256), st, a);
  else GDR_LAUNCH("scan_state", (scan_kernel<T, VB, MODE_STATE>), grid, dim3(256), st, a);
}

template <typename T>
void launch_scan(const Plan& pl, ScanArgs a, int mode, hipStream_t st) {
  if (pl.vb == 2) launch_scan_vb<T, 2>(pl, a, mode, st);
  else launch_scan_vb<T, 1>(pl, a, mode, st);
}
template void launch_scan<__bf16>(const Plan&, ScanArgs, int, hipStream_t);
template void launch_scan<_Float16>(const Plan&, ScanArgs, int, hipStream_t);

gdr_status launch_fwd(const gdr_problem* p, const Plan& pl, const void* q, const void* k,
                      const void* v, const void* g, const void* beta, const float* h0,
                      float* gcum, void* A, void* o, void* h, float* trans, float* ht, void* ws,
                      hipStream_t st, void* qn, void* kn, float* qinv, float* kinv) {
  if ((qn || kn || qinv || kinv) && (!qn || !kn || !qinv || !kinv || p->use_qk_l2norm)) {
    set_error("unit rows are kept with both norms, on a problem that does not normalise");
    return GDR_ERR_ARG;
  }
  char* wp = reinterpret_cast<char*>(ws);
  const int32_t* offs = nullptr;
  const int32_t* order = nullptr;
  if (p->cu_seqlens_dev) {
    int32_t* o32 = reinterpret_cast<int32_t*>(wp);
    wp += align256(sizeof(int32_t) * (size_t)(pl.N + 1));
    int32_t* r32 = reinterpret_cast<int32_t*>(wp);
    wp += align256(sizeof(int32_t) * (size_t)pl.N);
    GDR_LAUNCH("chunk_offsets", chunk_offsets_kernel, dim3(1), dim3(256), st, p->cu_seqlens_dev,
               pl.N, o32, r32);
    offs = o32;
    order = r32;
  }
  FwdArgs fa;
  fa.q = q; fa.k = k; fa.v = v; fa.g = g; fa.beta = beta; fa.h0 = h0; fa.gcum = gcum;
  fa.A = A; fa.o = o; fa.h = h; fa.ht = ht;
  fa.cu = p->cu_seqlens_dev; fa.offs = offs;
  fa.N = pl.N; fa.T = p->T; fa.Hq = p->Hq; fa.Hv = p->Hv; fa.nc_dense = pl.nc_dense;
  fa.g_dtype = (int)p->g_dtype; fa.scale = p->scale; fa.svf = p->state_v_first ? 1 : 0;
  fa.qk_norm = p->use_qk_l2norm ? 1 : 0;
  fa.beta_mode = (p->beta_sigmoid ? 1 : 0) | (p->neg_eigval ? 2 : 0);
  fa.gate_A_log = p->use_gate ? p->gate_A_log : nullptr;
  fa.gate_dt_bias = p->use_gate ? p->gate_dt_bias : nullptr;
  fa.qn = qn; fa.kn = kn; fa.qinv = qinv; fa.kinv = kinv;
  if (qn) fa.qk_norm = 1;  // fwd_prep normalises and keeps the rows; the scans read them

  ScanArgs sa;
  memset(&sa, 0, sizeof(sa));
  sa.q = qn ? qn : q; sa.k = kn ? kn : k;
  sa.v = v; sa.beta = beta; sa.gcum = gcum; sa.A = A; sa.h0 = h0;
  sa.o = o; sa.h = h; sa.ht = ht; sa.trans = trans;
  sa.cu = p->cu_seqlens_dev; sa.offs = offs; sa.order = order;
  sa.N = pl.N; sa.T = p->T; sa.Hq = p->Hq; sa.Hv = p->Hv; sa.nc_dense = pl.nc_dense;
  sa.P = 1; sa.nvs = 1;
  sa.scale = p->scale; sa.svf = fa.svf; sa.h_svf = fa.svf;
  sa.h_vm = p->h_packed ? 1 : 0;
  sa.qk_norm = p->use_qk_l2norm ? 1 : 0;
  sa.beta_mode = fa.beta_mode;
  sa.seg_out = nullptr; sa.seg_start = nullptr;
  sa.reverse = 0;
  if (pl.cp > 1) {
    const size_t units = (size_t)pl.N * p->Hv;
    const size_t KV = (size_t)kDim * kDim;
    sa.seg_out = reinterpret_cast<float*>(wp);
    wp += align256(units * pl.cp * 2 * KV * sizeof(float));
    sa.seg_start = reinterpret_cast<float*>(wp);
  }
  const int64_t pairs = (int64_t)pl.total_chunks * p->Hv;
  const dim3 gp = pairs <= INT32_MAX ? dim3((unsigned)pairs)
                                     : dim3((unsigned)pl.total_chunks, (unsigned)p->Hv);
  if (p->in_dtype == GDR_BF16) {
    if (pl.total_chunks > 0 && qn)
      GDR_LAUNCH("fwd_prep", (fwd_prep_kernel<__bf16, true>), gp, dim3(256), st, fa);
    else if (pl.total_chunks > 0)
      GDR_LAUNCH("fwd_prep", (fwd_prep_kernel<__bf16, false>), gp, dim3(256), st, fa);
    launch_scan<__bf16>(pl, sa, MODE_OUT, st);
  } else {
    if (pl.total_chunks > 0 && qn)
      GDR_LAUNCH("fwd_prep", (fwd_prep_kernel<_Float16, true>), gp, dim3(256), st, fa);
    else if (pl.total_chunks > 0)
      GDR_LAUNCH("fwd_prep", (fwd_prep_kernel<_Float16, false>), gp, dim3(256), st, fa);
    launch_scan<_Float16>(pl, sa, MODE_OUT, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("forward launch failed: %s", hipGetErrorString(e));
    return GDR_ERR_HIP;
  }
  return GDR_OK;
}

}  // namespace gdr

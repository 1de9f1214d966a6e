// gdr_device.h -- device-side building blocks for the gfx950 kernels.
//
// MFMA fragment conventions (v_mfma_f32_16x16x32_{bf16,f16}, wave64):
//   lane l = 16 * grp + col,  grp = l / 16 in [0, 4),  col = l % 16
//   A operand (16 x 32): lane holds A[col][k(grp, e)] for e in [0, 8)
//   B operand (32 x 16): lane holds B[k(grp, e)][col]
//   D/C (16 x 16 fp32):  lane holds D[4 * grp + e][col] for e in [0, 4)
// The hardware only needs A and B to agree on the k order, so two orders are
// used:
//   contiguous: k = 8 * grp + e
//   split:      k = 4 * grp + e (e < 4),  16 + 4 * grp + (e - 4) (e >= 4)
// The split order is exactly how two vertically stacked D tiles sit in a
// lane, so an fp32 accumulator pair becomes a B operand by a register-local
// conversion (pack_split) with no data movement.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

template <typename T>
struct VT;
template <>
struct VT<__bf16> {
  typedef bf16x8 x8;
  typedef bf16x4 x4;
};
template <>
struct VT<_Float16> {
  typedef f16x8 x8;
  typedef f16x4 x4;
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// fp32 16x16x4: A lane holds A[col][grp] (k = grp), B lane holds B[grp][col].
__device__ __forceinline__ f32x4 mfma16f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

template <typename T>
__device__ __forceinline__ float to_f(T x) {
  return (float)x;
}
template <typename T>
__device__ __forceinline__ T from_f(float x) {
  return (T)x;  // round to nearest even
}

// ---- operand fragments read from LDS -------------------------------------
// `base` points at element (row0, k0) of a row-major matrix with leading
// dimension ld (elements).  Rows are the 16 A-rows (or B-columns).

// contiguous k order: one 16-byte read
template <typename T>
__device__ __forceinline__ typename VT<T>::x8 frag_row(const T* base, int ld) {
  const int l = lane_id();
  return *reinterpret_cast<const typename VT<T>::x8*>(base + (l & 15) * ld + 8 * (l >> 4));
}

// split k order: two 8-byte reads
template <typename T>
__device__ __forceinline__ typename VT<T>::x8 frag_row_split(const T* base, int ld) {
  const int l = lane_id();
  const T* p = base + (l & 15) * ld + 4 * (l >> 4);
  typename VT<T>::x4 lo = *reinterpret_cast<const typename VT<T>::x4*>(p);
  typename VT<T>::x4 hi = *reinterpret_cast<const typename VT<T>::x4*>(p + 16);
  return typename VT<T>::x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Transposed fragment, split k order: the operand's k index runs down the
// ROWS of a row-major LDS matrix X[k][m] (m contiguous); `base` points at
// X[k0][m0].  Lane (grp, col) receives X[k0 + k(grp, e)][m0 + col].  Uses
// ds_read_b64_tr_b16: inside each 16-lane group, lane j gets element j % 4 of
// the 8-byte slot addressed by lane 4e + j / 4, for e = 0..3.
template <typename T>
__device__ __forceinline__ typename VT<T>::x8 frag_tr_split(const T* base, int ld) {
  const int l = lane_id();
  const int grp = l >> 4, j = l & 15;
  const T* p0 = base + (4 * grp + (j >> 2)) * ld + 4 * (j & 3);
  const T* p1 = p0 + 16 * ld;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  i16x8 r = i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename VT<T>::x8, r);
}

// Transposed fragment, contiguous k order.
template <typename T>
__device__ __forceinline__ typename VT<T>::x8 frag_tr(const T* base, int ld) {
  const int l = lane_id();
  const int grp = l >> 4, j = l & 15;
  const T* p0 = base + (8 * grp + (j >> 2)) * ld + 4 * (j & 3);
  const T* p1 = p0 + 4 * ld;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  i16x8 r = i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename VT<T>::x8, r);
}

// Four rows of one column in D-tile order: lane (grp, col) receives
// X[row0 + 4 grp + e][col0 + col], e = 0..3, from a row-major LDS matrix with
// one ds_read_b64_tr_b16 (lane j of group grp addresses row row0 + 4 grp + j/4,
// columns col0 + 4 (j % 4) ..).
template <typename T>
__device__ __forceinline__ f32x4 frag_d4(const T* X, int ld, int row0, int col0) {
  const int l = lane_id();
  const int grp = l >> 4, j = l & 15;
  const T* p = X + (row0 + 4 * grp + (j >> 2)) * ld + col0 + 4 * (j & 3);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const typename VT<T>::x4 v = __builtin_bit_cast(typename VT<T>::x4, r);
  return f32x4{to_f(v[0]), to_f(v[1]), to_f(v[2]), to_f(v[3])};
}

// Store a D tile transposed: lane (grp, col) writes its four rows as four
// consecutive elements of row col0 + col of Xt (Xt[c][r] = X[r][c]).
template <typename T>
__device__ __forceinline__ void store_d4_t(T* Xt, int ld, int row0, int col0, f32x4 v) {
  const int l = lane_id();
  const int grp = l >> 4, col = l & 15;
  typename VT<T>::x4 o{from_f<T>(v[0]), from_f<T>(v[1]), from_f<T>(v[2]), from_f<T>(v[3])};
  *reinterpret_cast<typename VT<T>::x4*>(Xt + (col0 + col) * ld + row0 + 4 * grp) = o;
}

// dot product of two registers of eight packed 16-bit values, in fp32
template <typename T>
__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  const typename VT<T>::x8 x = __builtin_bit_cast(typename VT<T>::x8, a);
  const typename VT<T>::x8 y = __builtin_bit_cast(typename VT<T>::x8, b);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += to_f(x[e]) * to_f(y[e]);
  return s;
}

// Two stacked fp32 D tiles (rows 0..15 and 16..31 of a 32-row block) become a
// split-order B operand (k = the 32 rows).
template <typename T>
__device__ __forceinline__ typename VT<T>::x8 pack_split(f32x4 top, f32x4 bot) {
  return typename VT<T>::x8{from_f<T>(top[0]), from_f<T>(top[1]), from_f<T>(top[2]),
                            from_f<T>(top[3]), from_f<T>(bot[0]), from_f<T>(bot[1]),
                            from_f<T>(bot[2]), from_f<T>(bot[3])};
}

// ---- global <-> LDS tile copies -------------------------------------------
// Copy `rows` valid rows (the rest zero-filled, up to 64) of a row-major tile
// of `cols` elements (cols % 8 == 0) whose rows sit `gstride` elements apart
// in global memory into LDS with leading dimension ld.  16-byte transfers,
// all threads of the block cooperate.
template <typename T, int NT>
__device__ __forceinline__ void tile_to_lds(T* lds, int ld, const T* g, int64_t gstride, int rows,
                                            int cols) {
  const int per_row = cols / 8;
  const int total = 64 * per_row;
  for (int x = threadIdx.x; x < total; x += NT) {
    const int r = x / per_row, c8 = (x % per_row) * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < rows) val = *reinterpret_cast<const uint4*>(g + r * gstride + c8);
    *reinterpret_cast<uint4*>(lds + r * ld + c8) = val;
  }
}

// ---- staggered 64 x 128 tiles -----------------------------------------------
// Rows of a 64 x 128 tile of 16-bit values are contiguous (256 bytes) but
// start at staggered offsets: row r begins 16 * U(r) bytes past 256 * r, with
// U(r) = 2 (r % 4) + 8 q + (q >= 2) + 32 (r / 16), q = (r / 4) % 4.  U grows
// with r, so rows never overlap.  Modulo the 256-byte bank width the
// 16-byte shifts of rows 0..15 are all different (operand rows read at one
// column hit distinct banks) and four consecutive rows are shifted by 32
// bytes each, so the 4 row x 32 byte reads of the transposing load cover all
// banks once; with a uniform 272-byte stride those reads collide two ways.
__device__ __forceinline__ int qk_row(int r) {
  const int q = (r >> 2) & 3;
  return 128 * r + 8 * (2 * (r & 3) + 8 * q + (q >> 1) + 32 * (r >> 4));
}
constexpr int QK_TILE = 128 * 64 + 8 * 128;  // elements, >= qk_row(63) + 128

// Operand rows r0 + (lane % 16) (r0 a multiple of 16), split k order (k0 a
// multiple of 32).
template <typename T>
__device__ __forceinline__ typename VT<T>::x8 frag_row_split_q(const T* X, int r0, int k0) {
  const int l = lane_id();
  const T* p = X + qk_row(l & 15) + (r0 >> 4) * qk_row(16) + k0 + 4 * (l >> 4);
  typedef typename VT<T>::x4 x4;
  const x4 lo = *reinterpret_cast<const x4*>(p);
  const x4 hi = *reinterpret_cast<const x4*>(p + 16);
  return typename VT<T>::x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Operand rows r0 + (lane % 16), contiguous k order (8 elements from
// k0 + 8 * (lane / 16)).
template <typename T>
__device__ __forceinline__ typename VT<T>::x8 frag_row_q(const T* X, int r0, int k0) {
  const int l = lane_id();
  const T* p = X + qk_row(l & 15) + (r0 >> 4) * qk_row(16) + k0 + 8 * (l >> 4);
  return *reinterpret_cast<const typename VT<T>::x8*>(p);
}

// Transposed operand (split k order): k runs down rows k0 .. k0 + 31 of the
// tile (k0 a multiple of 32), the operand's columns are m0 .. m0 + 15.
template <typename T>
__device__ __forceinline__ typename VT<T>::x8 frag_tr_split_q(const T* X, int k0, int m0) {
  const int l = lane_id(), j = l & 15;
  const T* p = X + qk_row(4 * (l >> 4) + (j >> 2)) + (k0 >> 4) * qk_row(16) + m0 + 4 * (j & 3);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + qk_row(16)));
  return __builtin_bit_cast(typename VT<T>::x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// frag_d4 on a staggered tile (row0 a multiple of 16).
template <typename T>
__device__ __forceinline__ f32x4 frag_d4_q(const T* X, int row0, int col0) {
  const int l = lane_id();
  const int grp = l >> 4, j = l & 15;
  const T* p = X + qk_row(4 * grp + (j >> 2)) + (row0 >> 4) * qk_row(16) + col0 + 4 * (j & 3);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const typename VT<T>::x4 v = __builtin_bit_cast(typename VT<T>::x4, r);
  return f32x4{to_f(v[0]), to_f(v[1]), to_f(v[2]), to_f(v[3])};
}

// ---- swizzled tiles, filled by LDS-direct loads -------------------------------
// A 16-byte buffer load to LDS (gfx950) writes the pieces fetched by a
// wave's 64 lanes to 1 KiB of consecutive LDS, lane by lane, so a tile
// filled that way has unpadded rows.  Bank conflicts are avoided instead by
// permuting the 16-byte pieces of each row: piece j of row r sits at
// position j ^ sw_piece(r).
//   64 x 128 (q, k; 256-byte rows): sw(r) = 2 (r % 8) + (r / 8) % 2.  It
//     takes every value over 16 aligned rows (a row operand reads one piece
//     of each of 16 rows) and sw / 2 every value over 8 aligned rows (a
//     transposing read takes two adjacent pieces, 32 bytes, of 8 rows).
//   64 x 64 (A, dO; 128-byte rows, two to 256 bytes): sw(r) =
//     2 ((r / 2) % 4) + (r / 8) % 2.  Over 16 aligned rows (r % 2, sw) takes
//     every value (row operands), and (r % 2, sw / 2) over 8 aligned rows
//     (transposing reads).
//   64 x 32 (32 value columns; 64-byte rows): sw(r) = 2 ((r / 4) % 2).  The
//     transposing reads take 32 bytes of 8 aligned rows; rows 4..7 land in the
//     other half of their 64 bytes.
template <int COLS>
__device__ __forceinline__ int sw_piece(int r) {
  static_assert(COLS == 128 || COLS == 64 || COLS == 32, "swizzled tile width");
  if (COLS == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
  if (COLS == 64) return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
  return ((r >> 2) & 1) << 1;
}

// element offset of (r, c) in a swizzled tile of COLS 16-bit columns
template <int COLS>
__device__ __forceinline__ int sw_off(int r, int c) {
  return COLS * r + 8 * ((c >> 3) ^ sw_piece<COLS>(r)) + (c & 7);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// s_waitcnt immediate that waits until at most n (< 64) vector memory
// operations of the wave are outstanding (the export and LDS counters are
// left alone)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt immediate that waits for the wave's LDS operations only
constexpr int lgkmcnt0_imm() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// Operand rows r0 + (lane % 16) (r0 a multiple of 16), split k order.
template <typename T, int COLS>
__device__ __forceinline__ typename VT<T>::x8 frag_row_split_w(const T* X, int r0, int k0,
                                                                int l = lane_id()) {
  const int r = r0 + (l & 15), c = k0 + 4 * (l >> 4);
  typedef typename VT<T>::x4 x4;
  const x4 lo = *reinterpret_cast<const x4*>(X + sw_off<COLS>(r, c));
  const x4 hi = *reinterpret_cast<const x4*>(X + sw_off<COLS>(r, c + 16));
  return typename VT<T>::x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Operand rows r0 + (lane % 16), contiguous k order.
template <typename T, int COLS>
__device__ __forceinline__ typename VT<T>::x8 frag_row_w(const T* X, int r0, int k0) {
  const int l = lane_id();
  return *reinterpret_cast<const typename VT<T>::x8*>(
      X + sw_off<COLS>(r0 + (l & 15), k0 + 8 * (l >> 4)));
}

// Transposed operand, split k order: k runs down rows k0 .. k0 + 31, the
// operand's columns are m0 .. m0 + 15 (as frag_tr_split).
template <typename T, int COLS>
__device__ __forceinline__ typename VT<T>::x8 frag_tr_split_w(const T* X, int k0, int m0,
                                                               int l = lane_id()) {
  const int j = l & 15;
  const int r = k0 + 4 * (l >> 4) + (j >> 2), c = m0 + 4 * (j & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(X + sw_off<COLS>(r, c)));
  const i16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(X + sw_off<COLS>(r + 16, c)));
  return __builtin_bit_cast(typename VT<T>::x8,
                            i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// frag_d4 on a swizzled tile (row0 a multiple of 16).
template <typename T, int COLS>
__device__ __forceinline__ f32x4 frag_d4_w(const T* X, int row0, int col0) {
  const int l = lane_id(), grp = l >> 4, j = l & 15;
  const int r = row0 + 4 * grp + (j >> 2), c = col0 + 4 * (j & 3);
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(X + sw_off<COLS>(r, c)));
  const typename VT<T>::x4 v = __builtin_bit_cast(typename VT<T>::x4, x);
  return f32x4{to_f(v[0]), to_f(v[1]), to_f(v[2]), to_f(v[3])};
}

// One wave copies a 64-row tile of COLS 16-bit columns into a swizzled LDS
// tile, one 16-byte LDS-direct buffer load per 1 KiB.  Row r of the tile is
// at byte r * gs of the range rs; pieces past the range's end read as zero.
// Completion is counted by the wave's vector-memory counter: the wave waits
// for it (s_waitcnt vmcnt) before a barrier hands the tile to other waves.
template <int COLS>
__device__ __forceinline__ void tile_dma(__amdgpu_buffer_rsrc_t rs, int gs, void* lds,
                                         int l = lane_id()) {
  constexpr int PR = COLS / 8;  // pieces per row, = instructions per tile
#pragma unroll
  for (int m = 0; m < PR; ++m) {
    const int s = 64 * m + l, r = s / PR, j = (s % PR) ^ sw_piece<COLS>(s / PR);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)((char*)lds + 1024 * m), 16, r * gs + 16 * j,
        0, 0, 0);
  }
}

// ---- packed states ------------------------------------------------------------
// The chunk-start states the forward keeps for the backward, the backward's
// recomputed states and its chunk end-state gradients are stored the way the
// scans hold them: per (chunk, value head) the 128 x 128 values as
// [V/16][K/32][64 lanes][8], where lane (grp, col) of block (vb, kb2) holds
// value column 16 vb + col at keys 32 kb2 + 4 grp + e (e < 4) and
// 32 kb2 + 16 + 4 grp + e - 4 (e >= 4): the split-order MFMA operand of the
// 32 x 16 block.  A wave stores a block as 64 x 16 contiguous bytes (with
// 8-byte pieces of value-major rows, the same bytes cost several times more).
// The 64-column half starting at value v0 is then the 16 KiB starting at
// element v0 * 128, as in a value-major layout.
__device__ __forceinline__ int packed_off(int vb, int kb2, int lane) {
  return ((vb * 4 + kb2) * 64 + lane) * 8;
}

// Register-staged tile copies, split in two so that the global loads of the
// next chunk can be in flight while the current chunk computes.  A 64-row
// tile of COLS elements is NT-thread cooperative; thread t holds 16-byte
// pieces x = t + i * NT (row x / (COLS/8), column (x % (COLS/8)) * 8).
template <int COLS, int NT>
struct TileRegs {
  static constexpr int PER_ROW = COLS / 8;
  static constexpr int N = (64 * PER_ROW) / NT;
  static_assert((64 * PER_ROW) % NT == 0, "tile must split evenly");
  uint4 r[N];
};

// Raw buffer resource over the bytes [base, base + bytes).  Raw buffer
// instructions check each access against that range: a load past the end
// returns zero and a store past the end is dropped, so the ragged last chunk
// of a sequence needs no per-row branches.  Offsets are 32-bit byte offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t rs, int off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, rs, off, 0, 0);
}

__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t rs, int off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, 0);
}

// Non-temporal stores (cache policy bit 1, nt): data the kernel writes and
// never reads back, so that it does not displace lines that other
// workgroups are about to read.
__device__ __forceinline__ void buf_store16_nt(__amdgpu_buffer_rsrc_t rs, int off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, rs, off, 0, 2);
}
__device__ __forceinline__ void buf_store8_nt(__amdgpu_buffer_rsrc_t rs, int off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, 2);
}

// Stores and loads with cache policy sc1: coherent at device scope across
// the XCDs' L2s (a store is complete, for the wave's vector memory counter,
// once it is visible to such loads from any CU).  For data handed from one
// workgroup to another inside a launch.
__device__ __forceinline__ void buf_store16_sc1(__amdgpu_buffer_rsrc_t rs, int off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, rs, off, 0, 16);
}
__device__ __forceinline__ void buf_store_u32_sc1(__amdgpu_buffer_rsrc_t rs, int off, unsigned v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, rs, off, 0, 16);
}
__device__ __forceinline__ unsigned buf_load_u32_sc1(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 16);
}

// Rows [0, rows) of the tile load; rows past that read as zero.  Row r of the
// tile starts r * gstride elements after g (gstride >= COLS).
// `t0` is the calling thread's index among the NT cooperating threads; AUX
// is the loads' cache policy (16: sc1, coherent across the XCDs' L2s).
template <typename T, int COLS, int NT, int AUX = 0>
__device__ __forceinline__ void tile_load(TileRegs<COLS, NT>& t, const T* g, int64_t gstride,
                                          int rows, int t0 = threadIdx.x) {
  constexpr int PR = TileRegs<COLS, NT>::PER_ROW;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(g, (int64_t)rows * gstride * (int64_t)sizeof(T));
  const int gs = (int)gstride * (int)sizeof(T);
#pragma unroll
  for (int i = 0; i < TileRegs<COLS, NT>::N; ++i) {
    const int x = t0 + i * NT;
    const int r = x / PR, c8 = (x % PR) * 8;
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, r * gs + c8 * (int)sizeof(T), 0, AUX);
    t.r[i] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

template <typename T, int COLS, int NT>
__device__ __forceinline__ void tile_store(T* lds, int ld, const TileRegs<COLS, NT>& t,
                                           int t0 = threadIdx.x) {
  constexpr int PR = TileRegs<COLS, NT>::PER_ROW;
#pragma unroll
  for (int i = 0; i < TileRegs<COLS, NT>::N; ++i) {
    const int x = t0 + i * NT;
    const int r = x / PR, c8 = (x % PR) * 8;
    *reinterpret_cast<uint4*>(lds + r * ld + c8) = t.r[i];
  }
}

// Store a 64 x 128 register tile into a staggered LDS tile (qk_row).
template <typename T, int NT>
__device__ __forceinline__ void tile_store_q(T* lds, const TileRegs<128, NT>& t,
                                             int t0 = threadIdx.x) {
#pragma unroll
  for (int i = 0; i < TileRegs<128, NT>::N; ++i) {
    const int x = t0 + i * NT;
    *reinterpret_cast<uint4*>(lds + qk_row(x >> 4) + 8 * (x & 15)) = t.r[i];
  }
}

// Store 64 value columns of a packed state (64 x 128, loaded 16 bytes per
// piece in storage order, piece x = t0 + i * NT) into a staggered LDS tile of
// value-major rows (row = value column, qk_row).
template <typename T, int NT>
__device__ __forceinline__ void tile_store_packed_q(T* lds, const TileRegs<128, NT>& t,
                                                    int t0 = threadIdx.x) {
#pragma unroll
  for (int i = 0; i < TileRegs<128, NT>::N; ++i) {
    const int x = t0 + i * NT;
    const int ln = x & 63, kb2 = (x >> 6) & 3, vbl = x >> 8;
    T* p = lds + qk_row(16 * vbl + (ln & 15)) + 32 * kb2 + 4 * (ln >> 4);
    *reinterpret_cast<uint2*>(p) = make_uint2(t.r[i].x, t.r[i].y);
    *reinterpret_cast<uint2*>(p + 16) = make_uint2(t.r[i].z, t.r[i].w);
  }
}

// LDS tile rows [0, rows) -> global, 16 bytes per store (stores of rows past
// `rows` fall outside the buffer range and are dropped); NTS: non-temporal.
template <typename T, int COLS, int NT, bool NTS = false>
__device__ __forceinline__ void tile_from_lds(T* g, int64_t gstride, const T* lds, int ld,
                                              int rows) {
  constexpr int PR = COLS / 8;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(g, (int64_t)rows * gstride * (int64_t)sizeof(T));
  const int gs = (int)gstride * (int)sizeof(T);
#pragma unroll
  for (int i = 0; i < (64 * PR) / NT; ++i) {
    const int x = threadIdx.x + i * NT;
    const int r = x / PR, c8 = (x % PR) * 8;
    const uint4 val = *reinterpret_cast<const uint4*>(lds + r * ld + c8);
    if (NTS) buf_store16_nt(rs, r * gs + c8 * (int)sizeof(T), val);
    else buf_store16(rs, r * gs + c8 * (int)sizeof(T), val);
  }
}

__device__ __forceinline__ float load_scalar(const void* p, int64_t idx, int dtype) {
  // dtype: 0 bf16, 1 fp16, 2 fp32
  if (dtype == 0) return (float)reinterpret_cast<const __bf16*>(p)[idx];
  if (dtype == 1) return (float)reinterpret_cast<const _Float16*>(p)[idx];
  return reinterpret_cast<const float*>(p)[idx];
}

__device__ __forceinline__ void store_scalar(void* p, int64_t idx, int dtype, float v) {
  if (dtype == 0) reinterpret_cast<__bf16*>(p)[idx] = (__bf16)v;
  else if (dtype == 1) reinterpret_cast<_Float16*>(p)[idx] = (_Float16)v;
  else reinterpret_cast<float*>(p)[idx] = v;
}

// P = lower_incl(Q K^T o exp(gamma_r - gamma_i)) for one 64-token chunk,
// written to LDS in the input dtype.  The ten 16x16 tiles on or below the
// diagonal are spread over the four waves (3, 3, 2, 2); the two tiles above
// the diagonal that the triangular products read, (0,1) and (2,3), are zeroed
// once by p_zero_tiles and never written again.  LAY gives the layout of the
// q and k tiles: 0 rows ldq apart, 1 staggered (qk_row), 2 swizzled (sw_off);
// ldq is used by the first only.
enum { LAY_PLAIN = 0, LAY_STAG = 1, LAY_SWZ = 2 };
template <typename T, int LAY = LAY_PLAIN>
__device__ __forceinline__ void p_tiles(const T* Qs, const T* Ks, int ldq, T* Ps, int ldp,
                                        const float* gam, int w) {
  const int l = lane_id(), grp = l >> 4, col = l & 15;
  // (row block, column block) per wave and slot, 4 bits each (rb * 4 + cb),
  // 16 bits per wave: w0 (0,0) (2,0) (3,3); w1 (1,0) (1,1) (3,0);
  // w2 (2,1) (2,2); w3 (3,1) (3,2).  Decoded with scalar shifts of a
  // wave-uniform index (a table in memory would cost a load per chunk).
  constexpr uint64_t code = 0x0000ull | (0x8ull << 4) | (0xFull << 8) |
                            ((0x4ull | (0x5ull << 4) | (0xCull << 8)) << 16) |
                            ((0x9ull | (0xAull << 4)) << 32) |
                            ((0xDull | (0xEull << 4)) << 48);
  const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    if (t == 2 && wu >= 2) break;
    const int x = (int)((code >> (16 * wu + 4 * t)) & 15);
    const int rb = x >> 2, cb = x & 3;
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (LAY == LAY_STAG)
        acc = mfma16(frag_row_q(Qs, 16 * rb, 32 * kk), frag_row_q(Ks, 16 * cb, 32 * kk), acc);
      else if (LAY == LAY_SWZ)
        acc = mfma16(frag_row_w<T, 128>(Qs, 16 * rb, 32 * kk),
                     frag_row_w<T, 128>(Ks, 16 * cb, 32 * kk), acc);
      else
        acc = mfma16(frag_row(Qs + 16 * rb * ldq + 32 * kk, ldq),
                     frag_row(Ks + 16 * cb * ldq + 32 * kk, ldq), acc);
    }
    const f32x4 gr = *reinterpret_cast<const f32x4*>(gam + 16 * rb + 4 * grp);
    const float gi = gam[16 * cb + col];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * rb + 4 * grp + e, i = 16 * cb + col;
      // masked entries take exp(-inf) = 0 (an unconditional exponential)
      const float pv = acc[e] * __expf((rb != cb || i <= r) ? gr[e] - gi : -INFINITY);
      Ps[r * ldp + i] = from_f<T>(pv);
    }
  }
}

template <typename T>
__device__ __forceinline__ void p_zero_tiles(T* Ps, int ldp) {
  const int tid = threadIdx.x;  // 2 tiles of 256 elements, any block size
  for (int x = tid; x < 512; x += blockDim.x) {
    const int t = x >> 8, e = x & 255;
    const int r = 16 * (2 * t) + (e >> 4), i = 16 * (2 * t + 1) + (e & 15);
    Ps[r * ldp + i] = from_f<T>(0.f);
  }
}

// ---- cross-lane sums on the VALU (no LDS round trips) ----------------------
// DPP moves within rows of 16 lanes: quad_perm [1,0,3,2] (0xB1) and
// [2,3,0,1] (0x4E), row_half_mirror (0x141), row_mirror (0x140).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a lane group (lanes with the same l / 16).  Each
// step adds a lane to its mirror partner, so all 16 lanes end with the
// bitwise-identical sum.
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// Sum over the 4 lane groups (lanes with the same l % 16): the gfx950 row
// swaps exchange 16-lane rows (then 32-lane halves) between two registers,
// and the sum of the swapped pair is lane l's value plus its partner's.
__device__ __forceinline__ float sum4g(float v) {
  const int x = __builtin_bit_cast(int, v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = __builtin_bit_cast(float, (int)p16[0]) + __builtin_bit_cast(float, (int)p16[1]);
  const int y = __builtin_bit_cast(int, v);
  const auto p32 = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return __builtin_bit_cast(float, (int)p32[0]) + __builtin_bit_cast(float, (int)p32[1]);
}

// ---- q / k L2 normalisation ------------------------------------------------
// The use_qk_l2norm_in_kernel option that the FLA backend pull request's
// dispatch passes through: q and k rows (one per token and head) are scaled
// to unit length over K, x / sqrt(sum x^2 + eps), in fp32 and rounded back
// to the input type before any product reads them.
constexpr float kQKNormEps = 1e-6f;

// Normalises every row of a 64 x 128 register tile in place.  Thread x holds
// 8 elements of row x / 16 and the 16 threads of a row are 16 aligned
// consecutive lanes, so the row's sum of squares is one 16-lane DPP sum
// (fixed order).  With `rinv`, 1 / sqrt(sum x^2 + eps) of row r goes to
// rinv[r].  Rows past the chunk end load as zeros and stay zero.
template <typename T, int NT>
__device__ __forceinline__ void l2norm_rows(TileRegs<128, NT>& t, float* rinv,
                                            int t0 = threadIdx.x) {
#pragma unroll
  for (int i = 0; i < TileRegs<128, NT>::N; ++i) {
    typename VT<T>::x8 x = __builtin_bit_cast(typename VT<T>::x8, t.r[i]);
    float f[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[e] = to_f(x[e]);
      ss += f[e] * f[e];
    }
    const float ri = rsqrtf(sum16(ss) + kQKNormEps);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = from_f<T>(f[e] * ri);
    t.r[i] = __builtin_bit_cast(uint4, x);
    const int xr = t0 + i * NT;
    if (rinv != nullptr && (xr & 15) == 0) rinv[xr >> 4] = ri;
  }
}

// ---- beta options ------------------------------------------------------------
// The beta the recurrence uses, from the beta input x, for the two options the
// FLA backend pull request's verifier names: bit 0 of `mode`
// (use_beta_sigmoid_in_kernel) takes the sigmoid of a logit, bit 1
// (allow_neg_eigval) doubles it, so that I - beta k k^T can have a negative
// eigenvalue.  beta_used_grad is its derivative d beta / dx.
__device__ __forceinline__ float beta_used(float x, int mode) {
  const float b = (mode & 1) ? 1.f / (1.f + __expf(-x)) : x;
  return (mode & 2) ? 2.f * b : b;
}
__device__ __forceinline__ float beta_used_grad(float x, int mode) {
  float d = 1.f;
  if (mode & 1) {
    const float s = 1.f / (1.f + __expf(-x));
    d = s * (1.f - s);
  }
  return (mode & 2) ? 2.f * d : d;
}

// The gate activation (use_gate): the log decay from the gate input x and the
// head's parameters, g = -e^{A_log} softplus(x + dt_bias), the decay of the
// Mamba-2 discretisation that Gated DeltaNet layers use.  softplus(z) =
// max(z, 0) + log1p(e^{-|z|}) keeps both tails finite; d g / d x =
// -e^{A_log} sigmoid(x + dt_bias).
__device__ __forceinline__ float gate_softplus(float z) {
  return fmaxf(z, 0.f) + log1pf(__expf(-fabsf(z)));
}
__device__ __forceinline__ float gate_log_decay(float x, float a_log, float bias) {
  return -__expf(a_log) * gate_softplus(x + bias);
}
__device__ __forceinline__ float gate_log_decay_grad(float x, float a_log, float bias) {
  return -__expf(a_log) / (1.f + __expf(-(x + bias)));
}

// Inclusive prefix sum over the 64 lanes of a wave (fixed combination order).
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float y = __shfl_up(x, off, 64);
    if (l >= off) x += y;
  }
  return x;
}

// Workgroups are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Renumber blocks so that consecutive logical blocks -- the column blocks and
// segments of one (sequence, head) that read the same q, k, A tiles -- run on
// the same XCD and share its L2.  Identity when the grid is not a multiple
// of 8.
__device__ __forceinline__ int xcd_block(int b, int nblocks) {
  if (nblocks & 7) return b;
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

// The (sequence, head) unit of hardware block b of a scan launch with nb
// blocks, per_unit of them per unit (its segments and column blocks), and
// the block's index sub within the unit.  The blocks of one unit run on one
// XCD (xcd_block).  Packed sequences of unequal length (order: the sequences
// by chunk count, longest first) also start the longest chains first: the
// XCDs take the units in rank order, rank k on XCD k % 8, so that when there
// are more blocks than CUs the short chains, not the long ones, wait for a
// free CU.
struct BlockPos {
  int unit, sub;
};
__device__ __forceinline__ BlockPos block_pos(const int32_t* order, int b, int nb, int per_unit,
                                              int Hv) {
  BlockPos r;
  if (order && nb % (8 * per_unit) == 0) {
    const int x = b & 7, y = b >> 3;
    const int k = (y / per_unit) * 8 + x;
    r.unit = order[k / Hv] * Hv + k % Hv;
    r.sub = y % per_unit;
  } else {
    const int L = xcd_block(b, nb);
    r.unit = L / per_unit;
    r.sub = L % per_unit;
  }
  return r;
}

// Where a (sequence, chunk) pair starts.  Dense batches: sequence n spans
// tokens [n*T, n*T + T).  Packed input: cu_seqlens.
struct SeqInfo {
  int64_t start, end;
};
__device__ __forceinline__ SeqInfo seq_info(const int32_t* cu, int n, int T) {
  SeqInfo s;
  if (cu) {
    s.start = cu[n];
    s.end = cu[n + 1];
  } else {
    s.start = (int64_t)n * T;
    s.end = s.start + T;
  }
  return s;
}

// Largest n in [0, N) with offs[n] <= c (offs non-decreasing, offs[0] = 0).
__device__ __forceinline__ int find_seq(const int32_t* offs, int N, int c) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= c) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

}  // namespace gdr

// Device-side building blocks shared by the gfx950 kernels of the chunked
// gated delta rule: element types, MFMA fragments, global/LDS fragment
// loaders and wave-wide scans.
//
// Fragment convention (one wave = 64 lanes, lane l, group g = l / 16):
//   a 16x16 product C += A * B over a 32-wide contraction slab takes, per lane,
//   8 elements of A's row (l % 16) and 8 elements of B's column (l % 16) whose
//   contraction indices are kmap(g, e), e = 0..7, the same map for A and B.
//   The accumulator holds C[4g + i][l % 16] in element i (the MFMA result
//   layout of v_mfma_f32_16x16x*).  Because the map only has to agree between
//   A and B, kernels pick it to suit their data: "row" fragments use
//   kmap = 8g + e (one 16-byte load), "chained" fragments use
//   kmap = 4g + e (e < 4), 16 + 4g + (e - 4) (e >= 4), which is exactly what
//   an accumulator of two stacked 16-row blocks holds, so an MFMA result feeds
//   the next MFMA's B operand without leaving registers.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define GDR_DEV __device__ __forceinline__

// ---------------------------------------------------------------- vectors
//
// Fragments and half-fragments are handled as whole vectors (element-wise
// conversions with __builtin_convertvector, concatenation with
// __builtin_shufflevector); the kernels never insert single bf16 lanes.

template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x4 v4; typedef bf16x8 v8; };
template <> struct Vec<float> { typedef f32x4 v4; typedef f32x8 v8; };
template <typename T> using v4_t = typename Vec<T>::v4;
template <typename T> using v8_t = typename Vec<T>::v8;

GDR_DEV f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
GDR_DEV f32x8 zero8() { return f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}; }

template <typename T> GDR_DEV f32x4 to_f32(v4_t<T> x) { return __builtin_convertvector(x, f32x4); }
template <typename T> GDR_DEV f32x8 to_f32(v8_t<T> x) { return __builtin_convertvector(x, f32x8); }
template <typename T> GDR_DEV v4_t<T> cvt4(f32x4 x) { return __builtin_convertvector(x, v4_t<T>); }
template <typename T> GDR_DEV v8_t<T> cvt8(f32x8 x) { return __builtin_convertvector(x, v8_t<T>); }

GDR_DEV f32x8 cat8(f32x4 lo, f32x4 hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }
GDR_DEV bf16x8 cat8(bf16x4 lo, bf16x4 hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

// ---------------------------------------------------------------- fragments

template <typename T> struct Frag {
  v8_t<T> v;
  GDR_DEV f32x8 f32() const { return to_f32<T>(v); }
  GDR_DEV static Frag make(f32x8 x) { Frag r; r.v = cvt8<T>(x); return r; }
  GDR_DEV static Frag raw(v8_t<T> x) { Frag r; r.v = x; return r; }
};

template <typename T> GDR_DEV Frag<T> frag_zero() { return Frag<T>::make(zero8()); }

// Two 4-element halves (as floats) -> one chained fragment.
template <typename T> GDR_DEV Frag<T> frag_from_halves(f32x4 lo, f32x4 hi) {
  return Frag<T>::make(cat8(lo, hi));
}

// acc += A * B over one 32-wide slab.  bf16: one v_mfma_f32_16x16x32_bf16.
// fp32: eight v_mfma_f32_16x16x4_f32; in step e each lane feeds its element e,
// which the instruction reads as contraction index g, so the slab is covered
// with the same kmap for A and B.
GDR_DEV void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
GDR_DEV void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// 16x16x16 fp32 product step used by the triangular solve: acc += A * B where
// lane l supplies A[l%16][4g + s] and B[4g + s][l%16] in step s.
GDR_DEV void mma16_f32(f32x4& acc, const float a[4], const float b[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
}

// Split x into a bf16 pair hi + lo with hi = bf16(x), lo = bf16(x - hi), so a
// product taken as hi*b + lo*b keeps about 16 mantissa bits of x.  For fp32
// fragments hi = x and lo is unused (kSplit is false).
template <typename T> struct SplitFrag {
  static constexpr bool kSplit = sizeof(T) == 2;
  Frag<T> hi, lo;
  GDR_DEV static SplitFrag make(f32x8 x) {
    SplitFrag s;
    s.hi = Frag<T>::make(x);
    if constexpr (kSplit) s.lo = Frag<T>::make(x - s.hi.f32());
    return s;
  }
};

// acc += A * B with A and / or B carried as hi + lo pairs (the lo*lo term is
// dropped: it sits below fp32 rounding of the accumulator).
template <typename T> GDR_DEV void mma_split(f32x4& acc, const SplitFrag<T>& a, const SplitFrag<T>& b) {
  mma(acc, a.hi, b.hi);
  if constexpr (SplitFrag<T>::kSplit) {
    mma(acc, a.hi, b.lo);
    mma(acc, a.lo, b.hi);
  }
}
template <typename T> GDR_DEV void mma_split(f32x4& acc, const Frag<T>& a, const SplitFrag<T>& b) {
  mma(acc, a, b.hi);
  if constexpr (SplitFrag<T>::kSplit) mma(acc, a, b.lo);
}
template <typename T> GDR_DEV void mma_split(f32x4& acc, const SplitFrag<T>& a, const Frag<T>& b) {
  mma(acc, a.hi, b);
  if constexpr (SplitFrag<T>::kSplit) mma(acc, a.lo, b);
}

// ---------------------------------------------------------------- memory

// 8 / 4 consecutive elements; p is 16-byte (8) / 8-byte (4) aligned for bf16,
// 16-byte aligned for fp32.
GDR_DEV Frag<bf16> ld8(const bf16* p) { return Frag<bf16>::raw(*reinterpret_cast<const bf16x8*>(p)); }
GDR_DEV Frag<float> ld8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return Frag<float>::raw(cat8(a, b));
}
GDR_DEV bf16x4 ld4raw(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
GDR_DEV f32x4 ld4raw(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
GDR_DEV f32x4 ld4f(const bf16* p) { return to_f32<bf16>(ld4raw(p)); }
GDR_DEV f32x4 ld4f(const float* p) { return ld4raw(p); }

GDR_DEV void st4(bf16* p, f32x4 x) { *reinterpret_cast<bf16x4*>(p) = cvt4<bf16>(x); }
GDR_DEV void st4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
GDR_DEV void st8(bf16* p, const Frag<bf16>& f) { *reinterpret_cast<bf16x8*>(p) = f.v; }
GDR_DEV void st8(float* p, const Frag<float>& f) {
  *reinterpret_cast<f32x4*>(p) = __builtin_shufflevector(f.v, f.v, 0, 1, 2, 3);
  *reinterpret_cast<f32x4*>(p + 4) = __builtin_shufflevector(f.v, f.v, 4, 5, 6, 7);
}

// Chained fragment from two 4-element pieces of one row.
GDR_DEV Frag<bf16> ld_chain(const bf16* lo, const bf16* hi) { return Frag<bf16>::raw(cat8(ld4raw(lo), ld4raw(hi))); }
GDR_DEV Frag<float> ld_chain(const float* lo, const float* hi) { return Frag<float>::raw(cat8(ld4raw(lo), ld4raw(hi))); }

// ------------------------------------------------------------ LDS transposes

// Transposed LDS read of 4 consecutive rows of one column of a row-major
// tile: the lane receives tile[row0 + m][col0 + (l % 16)], m = 0..3, where
// row0 and col0 are the same across each 16-lane group.  bf16 uses
// ds_read_b64_tr_b16: inside a 16-lane group lane i names 4 contiguous
// elements (a row of a 16 x 4 block) and lane l receives element l % 4 of the
// rows named by lanes l / 4 + 4m; so lane i names
// tile[row0 + i / 4][col0 + 4 * (i % 4)].  fp32 reads the four rows directly.
GDR_DEV bf16x4 lds_tr4(const bf16* tile, int pitch, int row0, int col0, int lane) {
  const int i = lane & 15;
  const bf16* p = tile + (row0 + (i >> 2)) * pitch + col0 + 4 * (i & 3);
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}
GDR_DEV f32x4 lds_tr4(const float* tile, int pitch, int row0, int col0, int lane) {
  const int c = col0 + (lane & 15);
  return f32x4{tile[row0 * pitch + c], tile[(row0 + 1) * pitch + c], tile[(row0 + 2) * pitch + c],
               tile[(row0 + 3) * pitch + c]};
}

// Fragment whose elements 0..3 are rows row_lo..row_lo+3 and 4..7 rows
// row_hi..row_hi+3 of column col0 + (l % 16).
template <typename T>
GDR_DEV Frag<T> lds_tr_frag(const T* tile, int pitch, int row_lo, int row_hi, int col0, int lane) {
  return Frag<T>::raw(cat8(lds_tr4(tile, pitch, row_lo, col0, lane), lds_tr4(tile, pitch, row_hi, col0, lane)));
}

// Rows r0 .. r0 + 3 of column c0 + l % 16 in fp32 -- the accumulator layout of
// a 16 x 16 block -- in one transposed read (r0 and c0 the same across each
// 16-lane group).
template <typename T>
GDR_DEV f32x4 lds_rows4(const T* tile, int pitch, int r0, int c0, int lane) {
  return to_f32<T>(lds_tr4(tile, pitch, r0, c0, lane));
}

GDR_DEV float to_float(bf16 x) { return (float)x; }
GDR_DEV float to_float(float x) { return x; }

// Store of two stacked 16-row accumulator blocks X (rows 4g..4g+3 of block 0)
// and Y (same rows of block 1), column l % 16, into the row of a transposed
// tile where the 32 rows are consecutive elements: v_permlane16_swap
// exchanges X of lane rows 1 / 3 with Y of rows 0 / 2, after which lane row g
// holds 8 consecutive elements starting at 16 (g & 1) + 8 (g >> 1) -- one
// 16-byte store per lane instead of two 8-byte ones.  `row` points at element
// 0 of the 32.
template <typename T>
GDR_DEV void st_pair(T* row, f32x4 X, f32x4 Y, int lane) {
  const int g = lane >> 4;
  if constexpr (sizeof(T) == 2) {
    const bf16x4 xb = cvt4<bf16>(X), yb = cvt4<bf16>(Y);
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 xu = __builtin_bit_cast(u32x2, xb), yu = __builtin_bit_cast(u32x2, yb);
    const auto s0 = __builtin_amdgcn_permlane16_swap(xu[0], yu[0], false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(xu[1], yu[1], false, false);
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 out = u32x4{s0[0], s1[0], s0[1], s1[1]};
    *reinterpret_cast<u32x4*>(row + 16 * (g & 1) + 8 * (g >> 1)) = out;
  } else {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 xu = __builtin_bit_cast(u32x4, X), yu = __builtin_bit_cast(u32x4, Y);
    u32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto sw = __builtin_amdgcn_permlane16_swap(xu[e], yu[e], false, false);
      a[e] = sw[0];
      b[e] = sw[1];
    }
    float* dst = reinterpret_cast<float*>(row) + 16 * (g & 1) + 8 * (g >> 1);
    *reinterpret_cast<u32x4*>(dst) = a;
    *reinterpret_cast<u32x4*>(dst + 4) = b;
  }
}

// Row-map fragment (contraction index 8 g + e) taken down a column of a
// row-major LDS tile: rows row0 + 8 g .. row0 + 8 g + 7 of column col0 + l % 16.
template <typename T>
GDR_DEV Frag<T> lds_col8(const T* tile, int pitch, int row0, int col0, int lane) {
  const int r = row0 + 8 * (lane >> 4);
  return lds_tr_frag(tile, pitch, r, r + 4, col0, lane);
}

// An fp32 operand tile in LDS.  For bf16 problems each value is kept as a
// bf16 pair hi + lo (about 16 mantissa bits), so MFMA operands come out as
// SplitFrag through the same 16-byte row reads and transposed column reads as
// plain bf16 tiles; for fp32 problems it is one float tile (lo unused).
template <typename T> struct FTile {
  static constexpr bool kSplit = sizeof(T) == 2;
  T* hi;
  T* lo;
  int pitch;
  GDR_DEV void put(int r, int c, float x) const {
    const T h = (T)x;
    hi[r * pitch + c] = h;
    if constexpr (kSplit) lo[r * pitch + c] = (T)(x - to_float(h));
  }
  // columns c .. c + 3 of row r (c a multiple of 4)
  GDR_DEV void put4(int r, int c, f32x4 x) const {
    const v4_t<T> h = cvt4<T>(x);
    *reinterpret_cast<v4_t<T>*>(hi + r * pitch + c) = h;
    if constexpr (kSplit) *reinterpret_cast<v4_t<T>*>(lo + r * pitch + c) = cvt4<T>(x - to_f32<T>(h));
  }
  GDR_DEV float get(int r, int c) const {
    float x = to_float(hi[r * pitch + c]);
    if constexpr (kSplit) x += to_float(lo[r * pitch + c]);
    return x;
  }
  // rows r0 .. r0 + 3 of column c0 + l % 16 (the accumulator layout)
  GDR_DEV f32x4 get4(int r0, int c0, int lane) const {
    f32x4 x = lds_rows4(hi, pitch, r0, c0, lane);
    if constexpr (kSplit) x += lds_rows4(lo, pitch, r0, c0, lane);
    return x;
  }
  // row r, contraction columns c0 + 8 g .. + 7
  GDR_DEV SplitFrag<T> row(int r, int c0, int lane) const {
    SplitFrag<T> f;
    const int o = r * pitch + c0 + 8 * (lane >> 4);
    f.hi = ld8(hi + o);
    if constexpr (kSplit) f.lo = ld8(lo + o);
    return f;
  }
  // column c0 + l % 16, contraction rows r0 + 8 g .. + 7
  GDR_DEV SplitFrag<T> col(int r0, int c0, int lane) const {
    SplitFrag<T> f;
    f.hi = lds_col8(hi, pitch, r0, c0, lane);
    if constexpr (kSplit) f.lo = lds_col8(lo, pitch, r0, c0, lane);
    return f;
  }
};

// An FTile of `rows` rows of pitch P at `base` (the lo tile, when there is
// one, follows the hi tile).
template <typename T, int P>
GDR_DEV FTile<T> ftile(char* base, int rows) {
  FTile<T> f;
  f.hi = reinterpret_cast<T*>(base);
  f.lo = FTile<T>::kSplit ? reinterpret_cast<T*>(base + (size_t)rows * P * sizeof(T)) : nullptr;
  f.pitch = P;
  return f;
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// fences global memory, which makes the compiler wait for every outstanding
// global load and store (s_waitcnt vmcnt(0)) and so drains software-pipelined
// prefetches; kernels whose waves only share data through LDS use this one.
GDR_DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- waves

// Inclusive prefix sum across the 64 lanes of a wave.
GDR_DEV float wave_incl_scan(float x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Cross-lane sums.  Inside each 16-lane row they stay in the vector ALU: DPP
// quad swaps, then the half-row and row mirrors (after each step every lane of
// a group holds its group's sum).  Across rows they use __shfl_xor.  Every
// lane of the wave must be active.
template <int CTRL> GDR_DEV float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N a power of two <= 64).
template <int N> GDR_DEV float lanes_sum_t(float x) {
  if constexpr (N >= 2) x += dpp_f<0xB1>(x);     // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_f<0x4E>(x);     // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_f<0x141>(x);    // row_half_mirror
  if constexpr (N >= 16) x += dpp_f<0x140>(x);   // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}
GDR_DEV float lanes_sum(float x, int n) {
  switch (n) {
    case 1: return x;
    case 2: return lanes_sum_t<2>(x);
    case 4: return lanes_sum_t<4>(x);
    case 8: return lanes_sum_t<8>(x);
    case 16: return lanes_sum_t<16>(x);
    case 32: return lanes_sum_t<32>(x);
    default: return lanes_sum_t<64>(x);
  }
}

// Sum over the four 16-lane groups (lanes l, l^16, l^32, l^48).
GDR_DEV float group4_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

constexpr float kL2Eps = 1e-6f;

// log2(e): gates kept in log2 units go straight to the hardware 2^x
constexpr float kLog2e = 1.4426950408889634f;
GDR_DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// beta as the operator uses it: the value passed, or its sigmoid when the
// caller passes logits.
GDR_DEV float beta_value(float x, int32_t logits) { return logits ? 1.f / (1.f + __expf(-x)) : x; }

// Compute units of one MI355X (8 XCDs x 32).
constexpr int64_t kNumCUs = 256;

// Workgroup index remap so that consecutive logical indices run on the same
// XCD (MI355X dispatches workgroups to its 8 XCDs round-robin); blocks that
// share input tiles then share an L2.
// Calls f(std::integral_constant<int, w>{}) for the wave index w in [0, N)
// (pass a scalar, e.g. __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)).
// Each wave then runs a body in which its index is a compile-time constant:
// per-wave block assignments and causal conditions fold away, so MFMA loops
// unroll without branches.  Shared-memory arrays belong outside the body (a
// __shared__ array declared in it would exist once per instantiation).
template <int N, typename F>
GDR_DEV void with_wave_index(int w, F&& f) {
  if constexpr (N > 1) {
    if (w == N - 1) {
      f(std::integral_constant<int, N - 1>{});
      return;
    }
    with_wave_index<N - 1>(w, f);
  } else {
    f(std::integral_constant<int, 0>{});
  }
}

GDR_DEV int64_t xcd_remap(int64_t bid, int64_t nblk) {
  if (nblk % 8 != 0) return bid;
  return (bid % 8) * (nblk / 8) + bid / 8;
}

// State-scan grids: the (sequence, value head, value tile) of a hardware
// block.  Without an order table, xcd_remap keeps a head's value tiles (which
// share w, k and q) on one XCD.  With seq_order (the sequences by decreasing
// chunk count), the (sequence, head) units are dealt round-robin over the 8
// XCDs in that order, each unit's tiles consecutive on its XCD: the longest
// scans start first and every XCD gets an equal share (longest-first list
// scheduling, which matters when a varlen batch mixes short and long
// sequences).
struct ScanUnit {
  int64_t n, j, vt;
};
GDR_DEV ScanUnit scan_unit(const int32_t* seq_order, int64_t N, int64_t HV, int64_t nvt) {
  const int64_t nblk = (int64_t)gridDim.x, b = (int64_t)blockIdx.x;
  if (seq_order == nullptr || (N * HV) % 8 != 0 || nblk != N * HV * nvt) {
    const int64_t bid = xcd_remap(b, nblk);
    return ScanUnit{bid / (nvt * HV), (bid / nvt) % HV, bid % nvt};
  }
  const int64_t x = b % 8, q = b / 8;
  const int64_t pos = x + 8 * (q / nvt);   // position in the ordered list of units
  return ScanUnit{(int64_t)seq_order[pos / HV], pos % HV, q % nvt};
}

// Chunk-parallel grids (one workgroup per chunk and head, launched as a 1-D
// grid of chunks x nheads): the heads of one chunk get consecutive logical
// indices on one XCD, so the per-token rows of g and beta (all heads of a
// token share one line) and a GVA group's key rows are fetched into one L2
// and shared instead of once per XCD.
struct ChunkHead {
  int64_t c, j;
};
GDR_DEV ChunkHead chunk_head(int64_t nheads) {
  const int64_t id = xcd_remap(blockIdx.x, (int64_t)gridDim.x);
  return ChunkHead{id / nheads, id % nheads};
}

}  // namespace gdr

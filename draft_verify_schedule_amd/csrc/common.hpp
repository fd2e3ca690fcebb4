// Device-side building blocks shared by the draft, schedule and verify
// kernels: bf16 loads, Philox4x32-10 uniforms, wave64 reductions and scans,
// softmax partial merging, and the MFMA fragment types of gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

namespace dspark {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Purposes of the per-decision uniforms.
constexpr uint32_t kPurposeDraft = 0;
constexpr uint32_t kPurposeAccept = 1;
constexpr uint32_t kPurposeResample = 2;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// Index of the calling wave within its workgroup, as a wave-uniform (scalar)
// value: derived from threadIdx.x the compiler would otherwise treat it as
// per-lane, and every buffer offset computed from it would need a
// readfirstlane loop around the load.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplications mixed with the other counter words and the round
// key; the key advances by the two Weyl constants between rounds.  Only the
// first output word is needed per decision.
__device__ __forceinline__ uint32_t philox_first_word(uint32_t c0, uint32_t c1, uint32_t c2,
                                                      uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint32_t lo0 = 0xD2511F53u * c0;
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

// Uniform in [0, 1) for decision (request, position, purpose) of `step`:
// the top 24 bits of the first Philox word, an exact float.
__device__ __forceinline__ float decision_uniform(uint64_t seed, uint64_t step, uint32_t request,
                                                  uint32_t position, uint32_t purpose) {
  const uint32_t w = philox_first_word((uint32_t)step, (uint32_t)(step >> 32), request,
                                       (position << 2) | purpose, (uint32_t)seed,
                                       (uint32_t)(seed >> 32));
  return (float)(w >> 8) * (1.0f / 16777216.0f);
}

// Raw buffer access: a buffer resource holds the base address and size; each
// load takes a 32-bit per-lane byte offset (VGPR) plus a wave-uniform byte
// offset (SGPR), so address arithmetic that is the same for the whole wave
// stays in scalar registers.  Offsets at or past the size read as zero.
// The fourth descriptor word is the gfx9-family data format (32-bit).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(rsrc_t r, uint32_t voffset, uint32_t soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voffset, (int)soffset, 0));
}

// The same load with the non-temporal cache policy (nt): for streams read
// once, so that they do not displace data that is read again (W2 across
// the draft positions and the residual pass's blocks).  Used only where each
// load instruction covers whole 128-byte lines (8 lanes x 16 bytes per
// line): where a line is assembled from several instructions (lanes 64 bytes
// apart, or the MFMA-layout loads of fp32 rows), each partial read then goes
// to memory again (measured: the fp32 residual pass 79 against 49 us with
// it; the row-statistics stream 175 against 111 us while each of its lanes
// read 64 contiguous bytes, 100 against 110 us once its load instructions
// covered whole lines).
__device__ __forceinline__ u32x4 buffer_load16_nt(rsrc_t r, uint32_t voffset, uint32_t soffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voffset, (int)soffset, 2));
}

__device__ __forceinline__ float2 buffer_load8(rsrc_t r, uint32_t voffset, uint32_t soffset) {
  typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
  const u32x2 d = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voffset, (int)soffset, 0));
  return make_float2(__uint_as_float(d[0]), __uint_as_float(d[1]));
}

// Raw-buffer range checking covers voffset + soffset: a load whose offset is
// at or past the resource size returns zeros without touching memory, and
// such a store is dropped.  Kernels use this as a branch-free mask: an offset
// of at least the resource size disables the access.
__device__ __forceinline__ void buffer_store8(rsrc_t r, float2 v, uint32_t voffset, uint32_t soffset) {
  typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
  const u32x2 d = {__float_as_uint(v.x), __float_as_uint(v.y)};
  __builtin_amdgcn_raw_buffer_store_b64(d, r, (int)voffset, (int)soffset, 0);
}

// The same 8-byte store issued as inline assembly, for loops that keep loads
// in flight.  The compiler's wait-count tracking treats a store pending next
// to loads as possibly completing out of order and then waits for all
// outstanding memory operations (vmcnt(0)) before using any load.  A store it
// does not see keeps its waits at "the loads issued after this one", which is
// still exact: loads complete in order, so at most N operations outstanding
// implies the load with N later loads has completed, whatever the stores do.
// The resource words are the four dwords of a raw buffer descriptor.
typedef int int4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4v raw_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return int4v{(int)(uint32_t)p, (int)(uint32_t)((p >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}
__device__ __forceinline__ void buffer_store8_untracked(int4v r, float2 v, uint32_t voffset, uint32_t soffset) {
  const double d = __hiloint2double((int)__float_as_uint(v.y), (int)__float_as_uint(v.x));
  asm volatile("buffer_store_dwordx2 %0, %1, %2, %3 offen" : : "v"(d), "v"(voffset), "s"(r), "s"(soffset));
}

__device__ __forceinline__ void buffer_store4_untracked(int4v r, float v, uint32_t voffset, uint32_t soffset) {
  asm volatile("buffer_store_dword %0, %1, %2, %3 offen" : : "v"(v), "v"(voffset), "s"(r), "s"(soffset));
}

// Hardware exp2 / log2 (v_exp_f32, v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---- wave64 helpers ------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Combine each lane's value with those of lanes l^16, l^32, l^48 (the same
// position in the other three 16-lane rows) using the gfx950 row-swap
// instructions, which run on the vector ALU instead of the LDS crossbar.
// Each swap of a register with itself hands every lane its own row's value
// and the partner row's value; the combine is symmetric, so which of the two
// comes first does not matter.
__device__ __forceinline__ void row_pair16(float v, float& a, float& b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(p[0]);
  b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void row_pair32(float v, float& a, float& b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(p[0]);
  b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void row_pair16(int v, int& a, int& b) {
  const auto p = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  a = (int)p[0];
  b = (int)p[1];
}
__device__ __forceinline__ void row_pair32(int v, int& a, int& b) {
  const auto p = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  a = (int)p[0];
  b = (int)p[1];
}
// max of two values that come from arithmetic or exchanges of such values
// (never a signalling NaN), as one v_max_f32: fmaxf would first quiet each
// exchanged operand with an extra instruction.  A quiet NaN operand yields the
// other operand, as fmaxf does.
__device__ __forceinline__ float max_arith(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float rows_max(float v) {
  float a, b;
  row_pair16(v, a, b);
  row_pair32(max_arith(a, b), a, b);
  return max_arith(a, b);
}
__device__ __forceinline__ float rows_sum(float v) {
  float a, b;
  row_pair16(v, a, b);
  row_pair32(a + b, a, b);
  return a + b;
}

// Exchanges within groups of 8 lanes on the DPP path (no LDS): xor 1 and
// xor 2 inside each quad, then lane i <-> 7 - i (the two quads of an 8-lane
// row half).  Three combining steps leave the 8-lane reduction in all 8 lanes.
__device__ __forceinline__ int dpp_q1(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_q2(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ int dpp_hm(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ float dpp_q1(float v) { return __int_as_float(dpp_q1(__float_as_int(v))); }
__device__ __forceinline__ float dpp_q2(float v) { return __int_as_float(dpp_q2(__float_as_int(v))); }
__device__ __forceinline__ float dpp_hm(float v) { return __int_as_float(dpp_hm(__float_as_int(v))); }
__device__ __forceinline__ float lanes8_max(float v) {
  v = fmaxf(v, dpp_q1(v));
  v = fmaxf(v, dpp_q2(v));
  return fmaxf(v, dpp_hm(v));
}
__device__ __forceinline__ float lanes8_sum(float v) {
  v += dpp_q1(v);
  v += dpp_q2(v);
  return v + dpp_hm(v);
}
// Lane i <-> 15 - i inside each 16-lane row: after an 8-lane reduction it
// joins the row's two halves.
__device__ __forceinline__ int dpp_mirror(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); }
__device__ __forceinline__ float dpp_mirror(float v) { return __int_as_float(dpp_mirror(__float_as_int(v))); }
// Whole-wave maximum and sum without LDS: 8 lanes on DPP, the row's halves by
// the row mirror, then the four rows by the row swaps.  Every lane ends with
// the result; the order of the additions is fixed.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = lanes8_max(v);
  v = fmaxf(v, dpp_mirror(v));
  return rows_max(v);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = lanes8_sum(v);
  v += dpp_mirror(v);
  return rows_sum(v);
}

// Inclusive prefix sum across the 64 lanes in lane order.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// fp64 version, used for the slice-level CDF (thousands of slice masses per
// row: an fp32 running sum would carry ~1e-6 relative error to the crossing).
__device__ __forceinline__ double wave_inclusive_scan(double v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// The same scans on the DPP path (no LDS): Hillis-Steele steps of 1, 2, 4, 8
// lanes inside each 16-lane row (row_shr, lanes without a source add 0), then
// the row totals carried across rows (row_bcast:15 into rows 1 and 3,
// row_bcast:31 into rows 2 and 3).  Exact sums are those of the LDS versions;
// rounding can differ in the last place (another association).
__device__ __forceinline__ uint32_t dpp_shr(uint32_t v, int n) {
  switch (n) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
    case 4: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
  }
}
__device__ __forceinline__ uint32_t dpp_bcast15(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_bcast31(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
}
__device__ __forceinline__ float wave_inclusive_scan_dpp(float v) {
#pragma unroll
  for (int n = 1; n <= 8; n <<= 1) v += __uint_as_float(dpp_shr(__float_as_uint(v), n));
  v += __uint_as_float(dpp_bcast15(__float_as_uint(v)));
  v += __uint_as_float(dpp_bcast31(__float_as_uint(v)));
  return v;
}
__device__ __forceinline__ double dpp_f64(double v, int step) {  // step 0..3: row_shr 1,2,4,8; 4: bcast15; 5: bcast31
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  if (step < 4) {
    lo = dpp_shr(lo, 1 << step);
    hi = dpp_shr(hi, 1 << step);
  } else if (step == 4) {
    lo = dpp_bcast15(lo);
    hi = dpp_bcast15(hi);
  } else {
    lo = dpp_bcast31(lo);
    hi = dpp_bcast31(hi);
  }
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_inclusive_scan_dpp(double v) {
#pragma unroll
  for (int step = 0; step < 6; ++step) v += dpp_f64(v, step);
  return v;
}

// Lowest lane whose predicate holds, or -1.
__device__ __forceinline__ int wave_first_lane(bool pred) {
  const unsigned long long m = __ballot(pred);
  return m ? __ffsll((long long)m) - 1 : -1;
}

// (max, sum of exp2(x - max)) pairs: merge two partial softmax statistics.
// A pair with max == -inf carries no mass.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  const float a = (m == -INFINITY) ? 0.0f : s * fast_exp2(m - M);
  const float b = (m2 == -INFINITY) ? 0.0f : s2 * fast_exp2(m2 - M);
  m = M;
  s = a + b;
}

// (max, first index) pairs for greedy decoding: larger value wins, lowest index on ties.
// An index of -1 marks an empty partial.
__device__ __forceinline__ void merge_argmax(float& m, int& idx, float m2, int idx2) {
  if (idx2 < 0) return;
  if (idx < 0 || m2 > m || (m2 == m && idx2 < idx)) {
    m = m2;
    idx = idx2;
  }
}

// (max, first index, second largest value) triples: the greedy statistics
// with the gap to the runner-up.  A value equal to the max at another index
// is a runner-up equal to the max (gap 0).  An index of -1 marks an empty
// partial.
__device__ __forceinline__ void merge_top2(float& m, int& idx, float& m2, float om, int oidx, float om2) {
  if (oidx < 0) return;
  if (idx < 0) {
    m = om;
    idx = oidx;
    m2 = om2;
    return;
  }
  if (om > m || (om == m && oidx < idx)) {
    m2 = fmaxf(m, om2);
    m = om;
    idx = oidx;
  } else {
    m2 = fmaxf(m2, om);
  }
}

// merge_argmax over the whole wave (the greedy statistics without the
// runner-up), every lane ending with the result: the same exchanges as
// wave_merge_top2.
__device__ __forceinline__ void wave_merge_argmax(float& m, int& idx) {
  merge_argmax(m, idx, dpp_q1(m), dpp_q1(idx));
  merge_argmax(m, idx, dpp_q2(m), dpp_q2(idx));
  merge_argmax(m, idx, dpp_hm(m), dpp_hm(idx));
  merge_argmax(m, idx, dpp_mirror(m), dpp_mirror(idx));
  float a, b;
  int ia, ib;
  row_pair16(m, a, b); row_pair16(idx, ia, ib);
  m = a; idx = ia;
  merge_argmax(m, idx, b, ib);
  row_pair32(m, a, b); row_pair32(idx, ia, ib);
  m = a; idx = ia;
  merge_argmax(m, idx, b, ib);
}

// merge_top2 over the whole wave, every lane ending with the result: 8 lanes
// on DPP, the row mirror, then the row swaps (merge_top2 is symmetric in its
// two operands, so both lanes of each exchange agree).
__device__ __forceinline__ void wave_merge_top2(float& m, int& idx, float& m2) {
  float om, om2;
  int oi;
  om = dpp_q1(m); oi = dpp_q1(idx); om2 = dpp_q1(m2);
  merge_top2(m, idx, m2, om, oi, om2);
  om = dpp_q2(m); oi = dpp_q2(idx); om2 = dpp_q2(m2);
  merge_top2(m, idx, m2, om, oi, om2);
  om = dpp_hm(m); oi = dpp_hm(idx); om2 = dpp_hm(m2);
  merge_top2(m, idx, m2, om, oi, om2);
  om = dpp_mirror(m); oi = dpp_mirror(idx); om2 = dpp_mirror(m2);
  merge_top2(m, idx, m2, om, oi, om2);
  float a, b, a2, b2;
  int ia, ib;
  row_pair16(m, a, b); row_pair16(idx, ia, ib); row_pair16(m2, a2, b2);
  m = a; idx = ia; m2 = a2;
  merge_top2(m, idx, m2, b, ib, b2);
  row_pair32(m, a, b); row_pair32(idx, ia, ib); row_pair32(m2, a2, b2);
  m = a; idx = ia; m2 = a2;
  merge_top2(m, idx, m2, b, ib, b2);
}

// Loads of 16 consecutive logits (bf16 or f32) starting at column n of a row,
// masking columns >= V with -inf.  VEC: the row base is 16-byte aligned and V
// is a multiple of the vector width, so each 16-byte vector is either entirely
// inside the row or entirely past its end.
template <typename T>
struct Logits16;

template <>
struct Logits16<uint16_t> {  // bf16 stored as raw bits
  template <bool VEC>
  __device__ __forceinline__ static void load(const uint16_t* __restrict__ row, int n, int V,
                                              float out[16]) {
    if (VEC) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = n + 8 * h;
        if (c < V) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(row + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            out[8 * h + 2 * e] = __uint_as_float(w[e] << 16);
            out[8 * h + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) out[8 * h + e] = -INFINITY;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        out[e] = (n + e < V) ? bf16_bits_to_f32(row[n + e]) : -INFINITY;
    }
  }
};

template <>
struct Logits16<float> {
  template <bool VEC>
  __device__ __forceinline__ static void load(const float* __restrict__ row, int n, int V,
                                              float out[16]) {
    if (VEC) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int c = n + 4 * h;
        if (c < V) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(row + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) out[4 * h + e] = w[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) out[4 * h + e] = -INFINITY;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) out[e] = (n + e < V) ? row[n + e] : -INFINITY;
    }
  }
};

__device__ __forceinline__ float load_logit(const uint16_t* row, int n) {
  return bf16_bits_to_f32(row[n]);
}
__device__ __forceinline__ float load_logit(const float* row, int n) { return row[n]; }

}  // namespace dspark

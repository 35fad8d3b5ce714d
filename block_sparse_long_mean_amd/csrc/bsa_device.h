// Device-side helpers shared by the libbsa kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define BSA_WAVE 64
#define BSA_DEV __device__ __forceinline__

// ---------------------------------------------------------------------------
// bfloat16 <-> float.  bf16 is stored as raw uint16 bits in memory.
// ---------------------------------------------------------------------------
BSA_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
// Round to nearest even (gfx950 converts in hardware).
BSA_DEV uint16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
BSA_DEV __bf16 f2bfh(float f) { return (__bf16)f; }

// 16 bytes = 8 bf16 from global/LDS
BSA_DEV u16x8 ld16(const void* p) { return *reinterpret_cast<const u16x8*>(p); }
BSA_DEV void st16(void* p, u16x8 v) { *reinterpret_cast<u16x8*>(p) = v; }
BSA_DEV bf16x8 as_bf(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }
BSA_DEV u16x8 as_u16(bf16x8 v) { return __builtin_bit_cast(u16x8, v); }

// Split a float into a bf16 head and a bf16 tail: x ~= hi + lo with
// |x - hi - lo| <= 2^-16 |x|.  Three bf16 MFMA passes (hi.hi + hi.lo + lo.hi)
// then give dot products close to fp32 accuracy.
BSA_DEV void split_bf(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// ---------------------------------------------------------------------------
// MFMA wrappers (layouts checked on the device):
//  16x16x32: A lane l -> row l%16, k 8*(l/16)+e;  B lane l -> col l%16, same k;
//            C lane l -> col l%16, rows 4*(l/16)+i.
//  32x32x16: A lane l -> row l%32, k 8*(l/32)+e;  B lane l -> col l%32, same k;
//            C lane l -> col l%32, row 8*(i/4) + 4*(l/32) + (i%4).
// ---------------------------------------------------------------------------
BSA_DEV f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
BSA_DEV f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Wave primitives
// ---------------------------------------------------------------------------
BSA_DEV int lane_id() { return threadIdx.x & 63; }
BSA_DEV uint64_t shfl_xor64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = (uint32_t)__shfl_xor((int)lo, m, 64);
  hi = (uint32_t)__shfl_xor((int)hi, m, 64);
  return ((uint64_t)hi << 32) | lo;
}
BSA_DEV uint64_t shfl64(uint64_t v, int src) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = (uint32_t)__shfl((int)lo, src, 64);
  hi = (uint32_t)__shfl((int)hi, src, 64);
  return ((uint64_t)hi << 32) | lo;
}
// Lane exchanges inside the 16-lane rows of a wave through DPP (a VALU
// operand modifier, no LDS round trip).  Controls: quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_shl:n = 0x100+n (lane i reads i+n),
// row_shr:n = 0x110+n (lane i reads i-n), row_ror:n = 0x120+n (lane i reads
// (i-n) mod 16).  Lanes whose source falls outside the row read 0 (so no
// prior value has to be copied into the destination first).
template <int CTRL>
BSA_DEV uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
BSA_DEV uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  return ((uint64_t)dpp32<CTRL>(hi) << 32) | dpp32<CTRL>(lo);
}
// value held by lane (li ^ M) of the same row, M in {1, 2, 4, 8}; li = lane % 16
template <int M>
BSA_DEV uint64_t row_xor64(uint64_t v, int li) {
  if constexpr (M == 1) return dpp64<0xB1>(v);
  else if constexpr (M == 2) return dpp64<0x4E>(v);
  else if constexpr (M == 8) return dpp64<0x128>(v);
  else {
    static_assert(M == 4, "row_xor64 takes 1, 2, 4 or 8");
    const uint64_t up = dpp64<0x104>(v);
    const uint64_t dn = dpp64<0x114>(v);
    return (li & 4) ? dn : up;
  }
}
// row_xor64 with a stride that is a constant once the caller's loops unroll
BSA_DEV uint64_t row_xor64_any(uint64_t v, int m, int li) {
  switch (m) {
    case 1: return row_xor64<1>(v, li);
    case 2: return row_xor64<2>(v, li);
    case 4: return row_xor64<4>(v, li);
    default: return row_xor64<8>(v, li);
  }
}

// 32-bit value held by lane (li ^ m) of the same 16-lane row, m in {1, 2, 4, 8}
BSA_DEV int row_xor32_any(int v, int m, int li) {
  const uint32_t u = (uint32_t)v;
  switch (m) {
    case 1: return (int)dpp32<0xB1>(u);
    case 2: return (int)dpp32<0x4E>(u);
    case 4: {
      // both exchanges run on every lane (a lane must not read a lane that a
      // branch has switched off), then each lane keeps its partner's value
      const uint32_t up = dpp32<0x104>(u), dn = dpp32<0x114>(u);
      return (int)((li & 4) ? dn : up);
    }
    default: return (int)dpp32<0x128>(u);
  }
}

// value held by lane `src` (wave-uniform)
BSA_DEV uint64_t readlane64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

BSA_DEV float wave_max(float v) {
  for (int m = 32; m > 0; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Maxima without the NaN quieting that fmaxf adds around every operand
// (v_max_f32 / v_max3_f32 as they are; the operands here are scores, finite
// or -inf).
BSA_DEV float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
BSA_DEV float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max of v over lanes l and l ^ 32: v_permlane32_swap exchanges the two
// halves of the wave in registers (no LDS round trip)
BSA_DEV float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
BSA_DEV float wave_sum(float v) {
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Top-k keys.  A candidate is packed as a 64-bit key whose unsigned order is
// (score ascending, block index descending): the larger key is the better
// candidate, so equal scores prefer the lower block index.  Key 0 is below
// every real key and marks an empty slot.
// ---------------------------------------------------------------------------
BSA_DEV uint32_t order_f32(float s) {
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// One side of a compare-exchange with partner o: the larger of the two when
// keep_max, else the smaller.  Selecting the partner on (v > o) != keep_max
// takes one compare and one select per 32-bit half, instead of forming both
// the maximum and the minimum and then choosing.  Equal operands are the same
// value either way.
BSA_DEV uint64_t cx_keep(uint64_t v, uint64_t o, bool keep_max) { return ((v > o) != keep_max) ? o : v; }
BSA_DEV int cx_keep_i32(int v, int o, bool keep_max) { return ((v > o) != keep_max) ? o : v; }

BSA_DEV uint64_t make_key(float s, uint32_t j) {
  return ((uint64_t)order_f32(s) << 32) | (uint64_t)(0xFFFFFFFFu - j);
}
BSA_DEV uint32_t key_index(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }

// Bitonic sort of 64*V keys held by one wave, element e = i*64 + lane in
// register v[i]; result descending in e.
template <int V>
BSA_DEV void wave_sort_desc(uint64_t (&v)[V]) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= 64 * V; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 64) {
        const int rs = stride >> 6;
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int j = i ^ rs;
          if (j > i) {
            const int e = i * 64 + lane;
            const bool desc = (e & size) == 0;
            const uint64_t a = v[i], b = v[j];
            const bool sw = desc ? (a < b) : (a > b);
            v[i] = sw ? b : a;
            v[j] = sw ? a : b;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          // strides inside a 16-lane row through DPP, wider ones through LDS
          const uint64_t o = stride < 16 ? row_xor64_any(v[i], stride, lane & 15) : shfl_xor64(v[i], stride);
          const int e = i * 64 + lane;
          const bool lower = (lane & stride) == 0;
          const bool desc = (e & size) == 0;
          const bool keep_max = (lower == desc);
          v[i] = cx_keep(v[i], o, keep_max);
        }
      }
    }
  }
}

// Ascending bitonic sort of 64 int32 values, one per lane.
BSA_DEV int wave_sort_asc_i32(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int o = stride < 16 ? row_xor32_any(v, stride, lane & 15) : __shfl_xor(v, stride, 64);
      const bool lower = (lane & stride) == 0;
      const bool asc = (lane & size) == 0;
      const bool keep_min = (lower == asc);
      v = cx_keep_i32(v, o, !keep_min);
    }
  }
  return v;
}

// Per-row candidate buffer in LDS: `cap` keys, a count and a threshold.
// Appending is open to every lane; compaction is done by one whole wave and
// keeps the best `topk` keys, sorted descending at the buffer's front.  Once
// `topk` keys are held, the threshold is the k-th best key and only strictly
// better candidates are appended.
template <int V>  // cap = 64 * V
BSA_DEV void row_compact(uint64_t* buf, int* cnt, uint64_t* thr, int topk) {
  const int lane = lane_id();
  const int c = *cnt;
  uint64_t v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    v[i] = e < c ? buf[e] : 0ull;
  }
  wave_sort_desc<V>(v);
  const int keep = c < topk ? c : topk;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    if (e < keep) buf[e] = v[i];
  }
  if (c >= topk && topk > 0) {
    const int e = topk - 1;
    uint64_t t = 0;
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (i == (e >> 6)) t = shfl64(v[i], e & 63);
    if (lane == 0) *thr = t;
  }
  if (lane == 0) *cnt = keep;
  __builtin_amdgcn_wave_barrier();
}

// XCD-aware remap: hardware hands workgroup w to XCD w % 8.  The logical id
// returned makes each XCD work through one contiguous range of logical ids,
// so that work items sharing data (consecutive logical ids) share an L2.
BSA_DEV int xcd_remap(int w, int n) {
  const int per = n >> 3, rem = n & 7, x = w & 7, i = w >> 3;
  return x * per + (x < rem ? x : rem) + i;
}

// Angle reduction for RoPE: a = pos * omega formed in double, reduced to
// [-pi, pi] in double, then sin/cos in float.
BSA_DEV void rope_sincos(int pos, double omega, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = (double)pos * omega;
  a -= two_pi * rint(a * (1.0 / two_pi));
  const float af = (float)a;
  sincosf(af, &s, &c);
}

// The same in double precision throughout.
BSA_DEV void rope_sincos_d(int pos, double omega, double& c, double& s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = (double)pos * omega;
  a -= two_pi * rint(a * (1.0 / two_pi));
  sincos(a, &s, &c);
}

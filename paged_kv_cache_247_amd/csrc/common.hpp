// Shared device helpers for the gfx950 paged-decode kernels: element types, 16-byte
// vector loads, and wave-level cross-lane reductions built on DPP and the gfx950 permlane
// swaps (no LDS round trip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

template <Dt> struct Elt;
template <> struct Elt<Dt::F32> { using T = float; static constexpr int bytes = 4; };
template <> struct Elt<Dt::F16> { using T = _Float16; static constexpr int bytes = 2; };
template <> struct Elt<Dt::BF16> { using T = uint16_t; static constexpr int bytes = 2; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Low / high element of a packed pair of 16-bit values, widened to fp32 (exact).
template <Dt DT> __device__ __forceinline__ float lo16(uint32_t w);
template <Dt DT> __device__ __forceinline__ float hi16(uint32_t w);
template <> __device__ __forceinline__ float lo16<Dt::BF16>(uint32_t w) { return bits_f(w << 16); }
template <> __device__ __forceinline__ float hi16<Dt::BF16>(uint32_t w) { return bits_f(w & 0xffff0000u); }
template <> __device__ __forceinline__ float lo16<Dt::F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <> __device__ __forceinline__ float hi16<Dt::F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Unpack N 32-bit words into fp32 elements (N words hold N fp32 or 2N 16-bit elements).
template <Dt DT, int N>
__device__ __forceinline__ void unpack_words(const uint32_t* w, float* out) {
  if constexpr (DT == Dt::F32) {
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = bits_f(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      out[2 * i] = lo16<DT>(w[i]);
      out[2 * i + 1] = hi16<DT>(w[i]);
    }
  }
}

// fp32 -> storage element, round to nearest even.
template <Dt DT> __device__ __forceinline__ typename Elt<DT>::T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<Dt::F32>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<Dt::F16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ uint16_t from_f32<Dt::BF16>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// KV tile loads. A tile is normally read once per decode call, so it is loaded with the
// non-temporal hint (streaming cache policy): on MI355X a random 4-8 KiB tile gather rises from
// about 5.9 to about 6.8 TB/s with it. When blocks are shared between sequences (a common
// prefix) ordinary cached loads let the shared tiles be served from the caches instead.
template <bool NT, class V>
__device__ __forceinline__ V load_kv(const char* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else return *reinterpret_cast<const V*>(p);
}

// Vector loads of B bytes (B = 4, 8 or a multiple of 16) of a KV tile into 32-bit words.
template <int B, bool NT>
__device__ __forceinline__ void load_words(const char* p, uint32_t* w) {
  static_assert(B == 4 || B == 8 || B % 16 == 0, "load width");
  if constexpr (B == 4) {
    w[0] = load_kv<NT, uint32_t>(p);
  } else if constexpr (B == 8) {
    u32x2 v = load_kv<NT, u32x2>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < B / 16; ++i) {
      u32x4 v = load_kv<NT, u32x4>(p + 16 * i);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  }
}

// ---------------------------------------------------------------- cross-lane exchange
// DPP controls (a "row" is 16 lanes).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each 16
constexpr int kRowRor8 = 0x128;       // lane i <- lane (i+8) mod 16, i.e. i^8 within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return bits_f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f_bits(x), CTRL, 0xF, 0xF, false));
}

// Pair rows 0<->1 and 2<->3 (lane i with lane i^16): returns op(x, x of the partner) in every
// lane. v_permlane16_swap exchanges the odd rows of its first operand with the even rows of its
// second; applied to (x, x) the two results hold each row pair's two values in every lane.
template <class Op>
__device__ __forceinline__ float across16(float x, Op op) {
  auto r = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  return op(bits_f(r[0]), bits_f(r[1]));
}
// Pair the two 32-lane halves (lane i with lane i^32) the same way with v_permlane32_swap.
template <class Op>
__device__ __forceinline__ float across32(float x, Op op) {
  auto r = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return op(bits_f(r[0]), bits_f(r[1]));
}

struct OpAdd { __device__ __forceinline__ float operator()(float a, float b) const { return a + b; } };
struct OpMax { __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// All-reduce over aligned groups of N consecutive lanes (N = 1..64, a power of two); every
// lane of a group ends with the group's result. Steps after the first two pair lanes whose
// groups already hold uniform values, so a mirror pairing is as good as an xor pairing.
template <int N, class Op>
__device__ __forceinline__ float group_reduce(float x, Op op) {
  if constexpr (N >= 2) x = op(x, dpp<kQuadXor1>(x));
  if constexpr (N >= 4) x = op(x, dpp<kQuadXor2>(x));
  if constexpr (N >= 8) x = op(x, dpp<kRowHalfMirror>(x));
  if constexpr (N >= 16) x = op(x, dpp<kRowMirror>(x));
  if constexpr (N >= 32) x = across16(x, op);
  if constexpr (N >= 64) x = across32(x, op);
  return x;
}

// All-reduce across the 64/N groups of N lanes (N = 8, 16, 32 or 64), pairing lanes at the
// same position inside their groups (lane i with i^8, i^16, i^32): lane i ends with op over
// the lanes i mod N, i mod N + N, ... of the whole wave.
template <int N, class Op>
__device__ __forceinline__ float cross_group_reduce(float x, Op op) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
  if constexpr (N <= 8) x = op(x, dpp<kRowRor8>(x));
  if constexpr (N <= 16) x = across16(x, op);
  if constexpr (N <= 32) x = across32(x, op);
  return x;
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

}  // namespace pkv

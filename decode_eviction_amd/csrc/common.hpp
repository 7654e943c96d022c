// Device helpers shared by the libkvsel kernels (gfx950, wave64).
//
// Matrix-core tiles.  All score kernels work on 32 x 32 output tiles of
// v_mfma_f32_32x32x16_bf16 (bf16 inputs) or v_mfma_f32_32x32x2_f32 (fp32
// inputs), accumulating in fp32.  A row of d elements is split into 16-byte
// chunks; lane l of a wave feeds row (l % 32) of its operand and takes the
// chunks 2j + (l / 32), j = 0 .. NC-1.  Any fixed lane->element assignment
// gives the same dot products as long as both operands use it, so A and B
// fragments are loaded by the same routine.  Output layout of a 32 x 32 tile
// (C = A.B^T over the chunked dimension): lane l, register i holds
//   column  l % 32  (the B-operand row)
//   row     8*(i/4) + 4*(l/32) + (i%4)  (the A-operand row).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// element-type tags
struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
};
struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;
};

template <typename E, int D>
struct Geo {
  static constexpr int kRowBytes = D * E::kBytes;
  static constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per row
  static constexpr int kNC = kChunks / 2;         // chunks per lane
  static constexpr int kLaneElems = kNC * E::kPerChunk;
};

template <int NC>
struct Frag {
  u32x4_t c[NC];
};

__device__ __forceinline__ u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// 4-byte loads through a buffer resource covering [base, base + bytes): an
// offset past the end reads 0, so a run of loads needs neither a branch nor a
// clamped index (one offset register and constant offsets serve all of them).
// The third word is the gfx9-family raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_ld32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

// s_waitcnt immediates (gfx9 encoding): wait until at most N vector memory
// operations of this wave are outstanding; LDS/scalar counters untouched.
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// 16 bytes per lane from a buffer straight into LDS: lane l of the wave
// writes bytes [16 l, 16 l + 16) from lds_wave_base (wave-uniform); offsets
// past the buffer's range write zeros.  Completion is counted by vmcnt.
__device__ __forceinline__ void buf_lds16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           (int)voff, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t buf_ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Row `row` of a row-major matrix whose rows are kRowBytes long; zero when
// !valid.  The load itself is unconditional (row 0 stands in for an invalid
// row) so that every load of a fragment is in flight before the first use.
template <typename E, int D>
__device__ __forceinline__ void load_frag(Frag<Geo<E, D>::kNC>& f, const char* base, long row,
                                          bool valid, int hf) {
  const char* p = base + (valid ? row : 0) * Geo<E, D>::kRowBytes + hf * 16;
#pragma unroll
  for (int j = 0; j < Geo<E, D>::kNC; ++j) f.c[j] = ld16(p + 32 * j);
  if (!valid) {
#pragma unroll
    for (int j = 0; j < Geo<E, D>::kNC; ++j) f.c[j] = zero4();
  }
}

// acc += A_frag . B_frag^T over all chunks
template <typename E, int NC>
__device__ __forceinline__ f32x16_t mfma_tile(const Frag<NC>& a, const Frag<NC>& b, f32x16_t acc);

template <>
__device__ __forceinline__ f32x16_t mfma_tile<BF16, 8>(const Frag<8>& a, const Frag<8>& b,
                                                       f32x16_t acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.c[j]),
                                                  __builtin_bit_cast(bf16x8_t, b.c[j]), acc, 0, 0, 0);
  return acc;
}
template <>
__device__ __forceinline__ f32x16_t mfma_tile<BF16, 4>(const Frag<4>& a, const Frag<4>& b,
                                                       f32x16_t acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.c[j]),
                                                  __builtin_bit_cast(bf16x8_t, b.c[j]), acc, 0, 0, 0);
  return acc;
}
// acc += one 16-byte chunk of A . the same chunk of B^T (the k-step a lane
// pair (l32, hf) covers in mfma_tile for that chunk index)
template <typename E>
__device__ __forceinline__ f32x16_t mfma_chunk(u32x4_t a, u32x4_t b, f32x16_t acc);
template <>
__device__ __forceinline__ f32x16_t mfma_chunk<BF16>(u32x4_t a, u32x4_t b, f32x16_t acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16_t mfma_chunk<F32>(u32x4_t a, u32x4_t b, f32x16_t acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc, 0, 0, 0);
  return acc;
}

template <int NC>
__device__ __forceinline__ f32x16_t mfma_tile_f32(const Frag<NC>& a, const Frag<NC>& b,
                                                  f32x16_t acc) {
#pragma unroll
  for (int j = 0; j < NC; ++j) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.c[j][e]),
                                                 __uint_as_float(b.c[j][e]), acc, 0, 0, 0);
  }
  return acc;
}
template <>
__device__ __forceinline__ f32x16_t mfma_tile<F32, 8>(const Frag<8>& a, const Frag<8>& b,
                                                      f32x16_t acc) {
  return mfma_tile_f32<8>(a, b, acc);
}
template <>
__device__ __forceinline__ f32x16_t mfma_tile<F32, 16>(const Frag<16>& a, const Frag<16>& b,
                                                       f32x16_t acc) {
  return mfma_tile_f32<16>(a, b, acc);
}

// Element e (0 .. kPerChunk-1) of chunk j of a fragment, widened to fp32.
template <typename E>
__device__ __forceinline__ float frag_elem(u32x4_t c, int e);
template <>
__device__ __forceinline__ float frag_elem<BF16>(u32x4_t c, int e) {
  uint32_t w = c[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}
template <>
__device__ __forceinline__ float frag_elem<F32>(u32x4_t c, int e) {
  return __uint_as_float(c[e]);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// w.lo * v.lo + w.hi * v.hi + acc for words holding two bf16 values (the
// products are exact in fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t v, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, v), acc, false);
}

// Squared norm of this lane's share of its row (add the partner lane's).
template <typename E, int NC>
__device__ __forceinline__ float frag_sumsq(const Frag<NC>& f);
template <>
__device__ __forceinline__ float frag_sumsq<BF16, 8>(const Frag<8>& f) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s0 = dot2_bf16(f.c[j][0], f.c[j][0], s0);
    s1 = dot2_bf16(f.c[j][1], f.c[j][1], s1);
    s0 = dot2_bf16(f.c[j][2], f.c[j][2], s0);
    s1 = dot2_bf16(f.c[j][3], f.c[j][3], s1);
  }
  return s0 + s1;
}
template <>
__device__ __forceinline__ float frag_sumsq<BF16, 4>(const Frag<4>& f) {
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s0 = dot2_bf16(f.c[j][0], f.c[j][0], s0);
    s1 = dot2_bf16(f.c[j][1], f.c[j][1], s1);
    s0 = dot2_bf16(f.c[j][2], f.c[j][2], s0);
    s1 = dot2_bf16(f.c[j][3], f.c[j][3], s1);
  }
  return s0 + s1;
}
template <int NC>
__device__ __forceinline__ float frag_sumsq_f32(const Frag<NC>& f) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf(__uint_as_float(f.c[j][e]), __uint_as_float(f.c[j][e]), s);
  return s;
}
template <>
__device__ __forceinline__ float frag_sumsq<F32, 8>(const Frag<8>& f) { return frag_sumsq_f32<8>(f); }
template <>
__device__ __forceinline__ float frag_sumsq<F32, 16>(const Frag<16>& f) { return frag_sumsq_f32<16>(f); }


// Dimension index of element e of chunk j for lane half hf.
template <typename E>
__device__ __forceinline__ int frag_dim(int j, int e, int hf) {
  return (2 * j + hf) * E::kPerChunk + e;
}

__device__ __forceinline__ float inv_norm_of(float sumsq) {
  return sumsq > 0.f ? 1.0f / sqrtf(sumsq) : 0.f;
}

// Row of register i in the 32x32 output tile for lane half hf.
__device__ __forceinline__ int tile_row(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }

// Inclusive prefix sum over the 64 lanes of a wave by DPP moves: shifts by
// 1, 2, 4 and 8 lanes inside each 16-lane row, then lane 15's row total
// added to rows 1 and 3 and lane 31's to rows 2 and 3.  Six VALU operations,
// no LDS round trip (a shuffle-up ladder takes six).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// The value of lane l ^ 32.  v_permlane32_swap exchanges the upper half of
// its first operand with the lower half of its second; with both set to v,
// the first result holds v of the lower half in every lane of the upper half
// and the second v of the upper half in the lower half.  A VALU exchange:
// no LDS round trip and no lane-index register (as a bpermute would need).
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

// Order-preserving map fp32 -> uint32 (larger float -> larger key); -0 -> +0.
__device__ __forceinline__ uint32_t score_key(float z) {
  uint32_t u = __float_as_uint(z + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Direct global->LDS copies (global_load_lds): lane l of the wave writes its
// 16 (or 4) bytes to LDS at base + 16 l (4 l); base must be wave-uniform.
// Written as inline assembly on purpose: when the compiler sees an LDS DMA it
// makes every later LDS read wait for all outstanding vector memory
// operations (it cannot tell ring slots apart), which would serialise a
// prefetch ring.  Callers order the copies themselves with an explicit
// s_waitcnt vmcnt and a barrier before reading what they wrote.  The
// instructions write no registers; their address registers are read at issue.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// m0 is named as clobbered for the reader; the compiler keeps no value of its
// own in m0 in the kernels that use these (checked in their assembly), and
// warns that a reserved register is listed.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_lds16(const void* g, const void* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_offset(lds_wave_base)))
               : "m0");
}
__device__ __forceinline__ void dma_lds4(const void* g, const void* lds_wave_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_offset(lds_wave_base)))
               : "m0");
}

#pragma clang diagnostic pop

// Device-scope relaxed stores and loads (gfx950: global stores/loads with
// sc1, written through to / read from the point where every XCD sees the
// same data).  Work-groups on different XCDs exchange small records with
// these instead of device-scope release/acquire fences, which write back or
// invalidate the whole L2 of an XCD.  A writer waits for its stores
// (vmem_done) before it signals, so a reader that has seen the signal reads
// the records it was waiting for.
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this wave's vector memory operations (stores included) are done
__device__ __forceinline__ void vmem_done() { __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); }

// ---- records exchanged between work-groups of one launch
//
// Bounded waits: a wait that runs this many polls sets bit 2 of the call's
// error word and gives up (the kernel still finishes).
constexpr int kSpinLimit = 1 << 20;

// The 32-bit tag of a head's words in one call: the head's epoch (a
// counter in the workspace that every call advances by one) plus the call's
// salt (a value the host draws for every launch: an even stride apart from
// the previous launch's, from a per-process random start), with the head
// index spread by an odd constant.  On one workspace, consecutive calls
// move the tag by the stride plus one (odd), so the last 2^32 calls' tags
// all differ and words an earlier call left behind never pass for this
// call's; graph replays (same salt) move it by one.  A workspace whose
// memory held other data (its epoch words overwritten, for instance with
// zeros) still gets a new tag from the salt.
__device__ __forceinline__ uint32_t head_tag(uint64_t ep, long head, uint32_t salt) {
  return salt + (uint32_t)ep + (uint32_t)head * 0x85ebca6bu;
}

// A 64-bit word holding a 32-bit value (low half) and a call's tag (high half).
__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t v) { return ((uint64_t)tag << 32) | v; }

// The value of the tagged word at `at`, read once as w: polled again until
// its tag is there (at most kSpinLimit times; then bit 2 of *err, if given).
__device__ __forceinline__ uint32_t untag_w(const uint64_t* at, uint64_t w, uint32_t tag, int32_t* err) {
  for (int it = 0; (uint32_t)(w >> 32) != tag; ++it) {
    if (it == kSpinLimit) {
      if (err) atomicOr(err, 4);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    w = ld_dev(at);
  }
  return (uint32_t)w;
}

// x * y rounded to fp32 on its own, never fused into a following add (the
// product is the value another kernel stores and reloads)
__device__ __forceinline__ float mul_unfused(float x, float y) {
#pragma clang fp contract(off)
  return x * y;
}

// 2^x on the transcendental unit (v_exp_f32)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Softmax statistics are kept in base 2: logits are pre-multiplied by
// log2(e)/sqrt(d), so exp(s - max) = 2^(t - max_t) with t = s * log2(e).
// Merge two (max, sum of 2^(t - max)) partials.
__device__ __forceinline__ void softmax_merge(float& m, float& s, float m2, float s2) {
  float mm = fmaxf(m, m2);
  if (mm == -INFINITY) {
    m = mm;
    s = 0.f;
    return;
  }
  // one explicit FMA, so that every kernel that merges the same partials
  // rounds them the same way, whatever the compiler would have fused
  s = fmaf(s, exp2_fast(m - mm), s2 * exp2_fast(m2 - mm));
  m = mm;
}

}  // namespace kvsel

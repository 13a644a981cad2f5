// Device-side helpers shared by the WKV7 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

constexpr int kWave = 64;

// DPP controls (GFX9 DPP16 encodings).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane l <- 7-l within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane l <- 15-l within each 16 lanes
constexpr int kDppRor4 = 0x124;       // lane l <- (l+4) mod 16 within the row
constexpr int kDppRor8 = 0x128;       // lane l <- (l+8) mod 16 within the row

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the LPR consecutive lanes (LPR in {4, 8, 16}, aligned groups);
// every lane of the group receives the sum.
template <int LPR>
__device__ __forceinline__ float group_allreduce(float x)
{
    static_assert(LPR == 4 || LPR == 8 || LPR == 16, "group size");
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    if constexpr (LPR >= 8) x += dpp<kDppHalfMirror>(x);
    if constexpr (LPR >= 16) x += dpp<kDppMirror>(x);
    return x;
}

// Exchange-and-add across lane bit 5: the result in lanes 0-31 is x summed
// over lane l and l^32; in lanes 32-63 it is y summed the same way
// (v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second).  The empty asm keeps the two results distinct:
// without it this compiler folds their sum into twice the first result.
__device__ __forceinline__ float swap_add32(float x, float y)
{
    auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                              __builtin_bit_cast(unsigned, y), false, false);
    unsigned lo = p[0], hi = p[1];
    asm volatile("" : "+v"(hi));
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// The same across lane bit 4 (v_permlane16_swap exchanges the odd 16-lane
// rows of its first operand with the even rows of its second): lanes with
// bit 4 clear get x summed over l and l^16, lanes with bit 4 set get y.
__device__ __forceinline__ float swap_add16(float x, float y)
{
    auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                              __builtin_bit_cast(unsigned, y), false, false);
    unsigned lo = p[0], hi = p[1];
    asm volatile("" : "+v"(hi));
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// The decay the Foundry page forms from its pre-activation omega in
// tm_pre_forward: w = exp(-c sigmoid(omega)), c = RX_WDECAY_COEFF = exp(-0.5).
// omega = -inf gives w = 1 (used to pad past the end of a sequence).
// Written with the hardware base-2 exponential and reciprocal (exp(x) =
// 2^(x log2 e); each within a few ulp): sigmoid(omega) = 1 / (1 +
// 2^(-omega log2 e)), w = 2^(-c log2(e) sigmoid(omega)).
constexpr float kDecayCoeff = 0.606530659712633424f;
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;
__device__ __forceinline__ float decay_from_pre(float omega)
{
    const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * omega));
    return __builtin_amdgcn_exp2f((-kDecayCoeff * kLog2e) * sg);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// Raw (untyped) buffer view of `bytes` bytes at `base`.  A buffer load at a
// per-lane byte offset >= bytes returns zeros and a store there is dropped,
// so the tail of a partial chunk needs no per-lane branch.  The range check
// applies to the per-lane offset only: every varying part of an address goes
// there, the scalar offset stays 0.  Word 3 is the gfx9 descriptor word for
// 32-bit untyped data.
constexpr int kRawBufferWord3 = 0x00020000;
using BufRsrc = __amdgpu_buffer_rsrc_t;

__device__ __forceinline__ BufRsrc raw_buffer(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRawBufferWord3);
}

// (the builtin's data operand is an unsigned int: pass the bits, not the
// value converted)
__device__ __forceinline__ void bstore(BufRsrc r, uint32_t off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, (int)off, 0, 0);
}

// 16-byte buffer load through the fp32 form of the intrinsic: this compiler
// lowers the integer 128-bit and 96-bit forms (__builtin_amdgcn_raw_buffer_
// load_b128 / _b96) to a single-dword load (seen in the generated code).
typedef float BufF4 __attribute__((ext_vector_type(4)));
__device__ BufF4 raw_buffer_load_f32x4(BufRsrc rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.ptr.buffer.load.v4f32");

__device__ __forceinline__ float4 bload4(BufRsrc r, uint32_t off)
{
    const BufF4 q = raw_buffer_load_f32x4(r, (int)off, 0, 0);
    return make_float4(q.x, q.y, q.z, q.w);
}

__device__ __forceinline__ uint2 bload2(BufRsrc r, uint32_t off)
{
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    const u2 q = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(q.x, q.y);
}

// One input element at element offset `elem` of a buffer, widened to fp32.
template <typename TIn>
__device__ __forceinline__ float bload1(BufRsrc r, uint32_t elem)
{
    if constexpr (sizeof(TIn) == 4)
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)(elem * 4), 0, 0));
    else
        return bf16_lo(__builtin_amdgcn_raw_buffer_load_b16(r, (int)(elem * 2), 0, 0));
}

// 4 consecutive input elements, loaded raw (fp32: 16 bytes, bf16: 8 bytes)
// and widened to fp32.
template <typename TIn>
struct InQuad {
    using raw = float4;
    __device__ static raw load(const TIn *p) { return *reinterpret_cast<const float4 *>(p); }
    __device__ static raw bload(BufRsrc r, uint32_t off) { return bload4(r, off); }
    __device__ static float4 f32(raw q) { return q; }
};

template <>
struct InQuad<uint16_t> {   // bf16 stored as raw 16-bit patterns
    using raw = uint2;
    __device__ static raw load(const uint16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
    __device__ static raw bload(BufRsrc r, uint32_t off) { return bload2(r, off); }
    __device__ static float4 f32(raw q)
    {
        return make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
    }
};

// Base pointers of NV input vectors with the same [B][T][H][N] layout.
template <typename TIn, int NV>
struct VecPtrs {
    const TIn *p[NV];
};

// Copies the per-step vectors of one (b, h) for steps [t0, t0 + nsteps) into
// registers (issue) and then into LDS (commit) as fp32, laid out
// lds[vec][step][n].  Steps past nsteps are not loaded.
//
// The vector index of every load is a compile-time constant and the wave
// that issues it is fixed per (vector, 64-unit chunk), so each base pointer
// is a kernel argument held in SGPRs: no pointer is ever chosen per lane
// (a per-lane choice gets lowered to a dependent load of the pointer).
template <typename TIn, int NV, int TB, int N, int NTHREADS>
struct Stager {
    static constexpr int kNW = NTHREADS / kWave;
    static constexpr int kUnitsPerVec = TB * N / 4;          // 4 elements per unit
    static_assert(kUnitsPerVec % 32 == 0, "staging granularity");
    // Chunks of 64 units per vector (a half chunk when 32 units: then two
    // vectors share one wave instruction, split by lane half).
    static constexpr int kCPV = kUnitsPerVec >= kWave ? kUnitsPerVec / kWave : 1;
    static constexpr bool kHalf = kUnitsPerVec < kWave;
    static constexpr int kSlots = kHalf ? (NV + 1) / 2 : NV * kCPV;   // chunk slots
    static constexpr int kPer = (kSlots + kNW - 1) / kNW;            // slots per wave
    typename InQuad<TIn>::raw buf[kPer];

    // Slot s holds vector q = s / kCPV, chunk s % kCPV (full chunks), or
    // vectors 2s and 2s+1 in the two lane halves (half chunks).  Wave w owns
    // slots w, w + kNW, ...
    __device__ __forceinline__ void issue(const VecPtrs<TIn, NV> &vec, int64_t base_t0,
                                          int64_t step_stride, int nsteps, int wave, int lane,
                                          unsigned mask = ~0u)
    {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
#pragma unroll
            for (int w = 0; w < kNW; ++w) {
                const int slot = k * kNW + w;
                if (slot >= kSlots || wave != w) continue;
                if constexpr (!kHalf) {
                    const int q = slot / kCPV;
                    if (!((mask >> q) & 1u)) continue;
                    const int unit = (slot % kCPV) * kWave + lane;
                    const int st = unit / (N / 4), n4 = unit % (N / 4);
                    if (st < nsteps)
                        buf[k] = InQuad<TIn>::load(vec.p[q] + base_t0 + st * step_stride + 4 * n4);
                } else {
                    const int q0 = 2 * slot;
                    const int unit = lane & 31;
                    const int st = unit / (N / 4), n4 = unit % (N / 4);
                    const TIn *src = vec.p[q0];
                    if (q0 + 1 < NV && lane >= 32) src = vec.p[q0 + 1];
                    const int qh = q0 + (lane >> 5);
                    const bool valid = st < nsteps && qh < NV && ((mask >> qh) & 1u);
                    if (valid)
                        buf[k] = InQuad<TIn>::load(src + base_t0 + st * step_stride + 4 * n4);
                }
            }
        }
    }

    __device__ __forceinline__ void commit(float *lds, int nsteps, int wave, int lane,
                                           unsigned mask = ~0u)
    {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
#pragma unroll
            for (int w = 0; w < kNW; ++w) {
                const int slot = k * kNW + w;
                if (slot >= kSlots || wave != w) continue;
                if constexpr (!kHalf) {
                    const int q = slot / kCPV;
                    if (!((mask >> q) & 1u)) continue;
                    const int unit = (slot % kCPV) * kWave + lane;
                    const int st = unit / (N / 4);
                    if (st < nsteps)
                        *reinterpret_cast<float4 *>(lds + 4 * (q * kUnitsPerVec + unit)) =
                            InQuad<TIn>::f32(buf[k]);
                } else {
                    const int q = 2 * slot + (lane >> 5);
                    const int unit = lane & 31;
                    const int st = unit / (N / 4);
                    if (st < nsteps && q < NV && ((mask >> q) & 1u))
                        *reinterpret_cast<float4 *>(lds + 4 * (q * kUnitsPerVec + unit)) =
                            InQuad<TIn>::f32(buf[k]);
                }
            }
        }
    }
};

// Direct HBM -> LDS staging (gfx950 global_load_lds_dwordx4) for fp32
// inputs: the same chunk ownership and LDS layout as Stager, but each wave
// instruction writes its 64 lanes' float4s straight into 1 KB of LDS, so no
// registers hold the block in flight.  The copies are complete after
// `s_waitcnt vmcnt(0)` (wait_dma) in the issuing wave; a barrier after that
// publishes them to the workgroup.
__device__ __forceinline__ void wait_dma()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// One lane's 16 bytes from global memory to LDS at lds_wave_base + lane * 16
// (the LDS byte address, which must be the same in every lane of the wave,
// goes through M0).  Written as inline
// asm so the compiler does not treat later LDS reads as possibly reading
// this copy: it would otherwise wait for every copy in flight before each
// LDS read.  Completion is awaited explicitly with wait_dma().  M0 is listed
// as clobbered; the compiler warns that it keeps no value of a reserved
// register across inline asm, which costs nothing here: nothing else in
// these kernels uses M0 (gfx950's LDS instructions do not take it), and in
// the generated code every write of M0 is this one, right before its copy.
__device__ __forceinline__ void dma16(const void *gsrc, const float *lds_wave_base)
{
    const unsigned m0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(const __attribute__((address_space(3))) float *)lds_wave_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gsrc), "s"(m0)
                 : "memory", "m0");
}

// The same with the global address split into a wave-uniform base (SGPRs)
// and a 32-bit per-lane byte offset, and the LDS byte address given as a
// wave-uniform value.
__device__ __forceinline__ void dma16_split(const void *gbase, unsigned lane_off, unsigned lds_addr)
{
    // (readfirstlane returns int: widen through uint32_t, not by sign)
    const uint64_t b = (uint64_t)(uintptr_t)gbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
    const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(lane_off), "s"(bs), "s"(m0)
                 : "memory", "m0");
}

template <int NV, int TB, int N, int NTHREADS>
struct DmaStager {
    using Geo = Stager<float, NV, TB, N, NTHREADS>;
    static constexpr int kNW = Geo::kNW, kUnitsPerVec = Geo::kUnitsPerVec, kCPV = Geo::kCPV;
    static constexpr bool kHalf = Geo::kHalf;
    static constexpr int kSlots = Geo::kSlots, kPer = Geo::kPer;

    __device__ __forceinline__ void issue(const VecPtrs<float, NV> &vec, int64_t base_t0,
                                          int64_t step_stride, int nsteps, int wave, int lane,
                                          float *lds, unsigned mask = ~0u)
    {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
#pragma unroll
            for (int w = 0; w < kNW; ++w) {
                const int slot = k * kNW + w;
                if (slot >= kSlots || wave != w) continue;
                if constexpr (!kHalf) {
                    const int q = slot / kCPV;
                    if (!((mask >> q) & 1u)) continue;
                    const int chunk = slot % kCPV;
                    const int unit = chunk * kWave + lane;
                    const int st = unit / (N / 4), n4 = unit % (N / 4);
                    if (st < nsteps)
                        dma16(vec.p[q] + base_t0 + st * step_stride + 4 * n4,
                              lds + 4 * (q * kUnitsPerVec + chunk * kWave));
                } else {
                    // lanes 0-31 carry vector 2*slot, lanes 32-63 the next one,
                    // which follows it in LDS
                    const int q0 = 2 * slot;
                    const int qh = q0 + (lane >> 5);
                    const int unit = lane & 31;
                    const int st = unit / (N / 4), n4 = unit % (N / 4);
                    const float *src = vec.p[q0];
                    if (q0 + 1 < NV && lane >= 32) src = vec.p[q0 + 1];
                    if (st < nsteps && qh < NV && ((mask >> qh) & 1u))
                        dma16(src + base_t0 + st * step_stride + 4 * n4,
                              lds + 4 * (q0 * kUnitsPerVec));
                }
            }
        }
    }
    __device__ __forceinline__ void commit(float *, int, int, int, unsigned = ~0u) {}
};

// The input stager for a dtype: DMA for fp32, registers (widening) for bf16.
template <typename TIn, int NV, int TB, int N, int NTHREADS>
struct InputStager {
    Stager<TIn, NV, TB, N, NTHREADS> st;
    static constexpr bool kDma = false;
    __device__ __forceinline__ void issue(const VecPtrs<TIn, NV> &vec, int64_t base_t0,
                                          int64_t step_stride, int nsteps, int wave, int lane,
                                          float *, unsigned mask = ~0u)
    {
        st.issue(vec, base_t0, step_stride, nsteps, wave, lane, mask);
    }
    __device__ __forceinline__ void commit(float *lds, int nsteps, int wave, int lane,
                                           unsigned mask = ~0u)
    {
        st.commit(lds, nsteps, wave, lane, mask);
    }
};
template <int NV, int TB, int N, int NTHREADS>
struct InputStager<float, NV, TB, N, NTHREADS> : DmaStager<NV, TB, N, NTHREADS> {
    static constexpr bool kDma = true;
};

}  // namespace wkv7

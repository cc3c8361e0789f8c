// entq_decode.hip -- gfx950 kernels of the interleaved rANS weight decoder.
//
// Weights stay compressed in device memory and are decoded into a buffer
// right before a transformer block's forward pass needs them [EntQuant,
// "Float8@2bits: Entropy Coding Enables Data-Free Model Compression",
// technical summary §2 "Decodificación en Tiempo de Inferencia"]; all of a
// block's matrices are decoded in one batch because a single matrix is too
// small to fill the GPU [DFloat11 write-up, "Descompresión por bloque
// transformer"].
//
// Mapping onto CDNA4: one wavefront owns one chunk; lane j of the wave holds
// the chunk's rANS state j, so one step of the wave decodes 64 consecutive
// symbols. Lanes whose state falls below 2^16 after the step read the next
// words of the chunk's shared word stream; a lane's position in it is the
// number of lower lanes that also read (ballot + mbcnt), and the wave's
// pointer advances by the popcount. The slot table of the tensor (4096 x 8
// bytes) sits in LDS, shared by the kWaves waves of a workgroup, which all
// decode chunks of that one tensor.
//
// Two kernels:
//  * decode_stream (the hot path): the word stream reaches LDS through a
//    per-wave ring fed by direct global->LDS loads issued far ahead of use,
//    so a renormalisation read is an LDS read; decoded bytes are staged in
//    LDS for a block of 8 steps and leave as 8 consecutive outputs per lane
//    (one 16-byte store for bf16), the fp32 row-scale multiply and the bf16
//    rounding fused into that store. Like DFloat11's kernel it stages output
//    on chip and writes it coalesced [DFloat11 write-up, "Kernels GPU de 2
//    etapas y metadatos auxiliares"], but rANS needs no counting pass: a
//    chunk's output position is known up front.
//  * decode_simple: one symbol per lane per step straight from global
//    memory; used for tensors whose chunk size or row length is not a
//    multiple of the 512-symbol block.
#include <hip/hip_runtime.h>

#include "entq.h"
#include "entq_internal.h"

namespace entq {
namespace {

__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint16_t bf16_bits(float v) {
    __bf16 b = (__bf16)v;  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, b);
}

// fl32(v * s) with v as the first operand: when both operands are NaN the
// hardware returns the first one (quieted), and the format defines the
// code's NaN to win. The compiler would otherwise put a uniform scale first.
__device__ __forceinline__ float mul_value_scale(float v, float s) {
    float r;
    asm("v_mul_f32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(s));
    return r;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to two bf16 (RNE) in one v_cvt_pk_bf16_f32, lo in bits 0..15.
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
    const float2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ void load_table(uint2 *T, const SlotEntry *tables, uint32_t tensor) {
    const uint4 *src = reinterpret_cast<const uint4 *>(tables + (size_t)tensor * kProbScale);
    uint4 *dst = reinterpret_cast<uint4 *>(T);
    for (uint32_t i = threadIdx.x; i < kProbScale / 2; i += kThreads) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// decode_simple
// ---------------------------------------------------------------------------

template <int MODE>
__global__ __launch_bounds__(kThreads) void decode_simple(
    const SlotEntry *__restrict__ tables, const DevTensor *__restrict__ tensors,
    const DevChunk *__restrict__ chunks, const DevTask *__restrict__ tasks, uint32_t task0,
    const uint8_t *__restrict__ blob, void *__restrict__ out, const float *__restrict__ scales,
    const uint8_t *__restrict__ signmant, int32_t *__restrict__ status) {
    __shared__ uint2 T[kProbScale];

    const DevTask task = tasks[task0 + blockIdx.x];
    const DevTensor td = tensors[task.tensor];
    load_table(T, tables, task.tensor);
    __syncthreads();

    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t lane = threadIdx.x & 63;
    if (wave >= task.n_chunks) return;
    const DevChunk ch = chunks[task.first_chunk + wave];
    const uint8_t *region = blob + ch.byte_offset;
    const uint16_t *words = reinterpret_cast<const uint16_t *>(region + kStateBytes);
    uint32_t x = reinterpret_cast<const uint32_t *>(region)[lane];
    const uint32_t n = ch.n_symbols;
    const uint32_t nw = ch.n_words;
    const uint32_t steps = (n + 63) >> 6;
    uint32_t p = 0;
    bool overrun = false;

    // row/column of this lane's symbol (element 64 t + lane of the chunk)
    const uint32_t cols = td.cols;
    uint64_t row = ch.scale_row;
    uint32_t col = ch.col0 + lane;
    if (MODE == kModeBf16)
        while (col >= cols) { col -= cols; ++row; }

    for (uint32_t t = 0; t < steps; ++t) {
        const uint32_t i = (t << 6) + lane;
        const bool active = i < n;
        uint32_t sym = 0;
        if (active) {
            const uint2 e = T[x & (kProbScale - 1)];
            x = __umul24(e.x, x >> kProbBits) + e.y;
            sym = e.x >> 24;
        }
        const bool need = active && x < kStateLow;
        const uint64_t mask = __ballot(need);
        if (need) {
            const uint32_t idx = p + lane_prefix(mask);
            if (idx < nw)
                x = (x << 16) | words[idx];
            else
                overrun = true;
        }
        p += (uint32_t)__popcll(mask);
        if (active) {
            const uint64_t o = ch.out_elem + i;
            if (MODE == kModeCodes) {
                static_cast<uint8_t *>(out)[o] = (uint8_t)sym;
            } else if (MODE == kModeBf16) {
                const float v = (td.kind == ENTQ_SYM_E4M3)
                                    ? __builtin_amdgcn_cvt_f32_fp8((int)sym, 0)
                                    : (float)(int8_t)sym;
                static_cast<uint16_t *>(out)[o] = bf16_bits(mul_value_scale(v, scales[row]));
            } else {
                const uint32_t s = signmant[o];
                static_cast<uint16_t *>(out)[o] =
                    (uint16_t)(((s & 0x80u) << 8) | (sym << 7) | (s & 0x7Fu));
            }
        }
        if (MODE == kModeBf16) {
            col += 64;
            while (col >= cols) { col -= cols; ++row; }
        }
    }
    const uint64_t bad_state = __ballot(x != kStateLow);
    const uint64_t bad_words = __ballot(overrun);
    if (status && lane == 0)
        status[ch.status_index] = (bad_words || p != nw) ? ENTQ_CHUNK_BAD_WORDS
                                  : (bad_state ? ENTQ_CHUNK_BAD_STATE : ENTQ_CHUNK_OK);
}

// ---------------------------------------------------------------------------
// decode_stream
// ---------------------------------------------------------------------------

// Word ring of one wave: kRingWords 16-bit words in LDS plus a mirror of its
// first kMirrorWords after the end, so that the up-to-64 words one step
// reads are contiguous without a wrap-around mask. It is refilled in units
// of kRingUnit words (64 lanes x 16 bytes, one direct global->LDS load) and
// kept at most kRingLead words ahead of the read pointer, which leaves one
// unit of room for the unit in flight.
constexpr uint32_t kRingWords = 2048;
constexpr uint32_t kMirrorWords = 64;
constexpr uint32_t kRingUnit = 512;
constexpr uint32_t kRingLead = kRingWords - kRingUnit;
static_assert(kRingLead >= 2 * kBlockSyms, "a block must find its words loaded a block early");

template <int MODE>
struct alignas(16) WaveLds {
    uint16_t ring[kRingWords + kMirrorWords];
    uint8_t stage[kBlockSyms];                               // decoded bytes of a block
    uint8_t sm[MODE == kModeSplit ? 2 : 1][MODE == kModeSplit ? kBlockSyms : 16];
};

// One 16-byte global->LDS load per active lane: lane l's bytes land at LDS
// address lds_base + 16 l. The compiler does not see this load, so it inserts
// no wait for it; the kernel waits with explicit vmcnt counts instead.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(gptr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// All vector-memory operations but the most recent `n` are complete. The asm
// form is invisible to the compiler's own wait insertion, which therefore
// never relaxes it.
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm1() { asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)p;
}

// Issues the load of words [first, first + kRingUnit) of the chunk into the
// ring (only lanes whose 16 bytes lie inside the chunk's region), and of the
// mirror when the unit starts the ring.
__device__ __forceinline__ void ring_fill(uint16_t *ring, const uint8_t *words_g, uint32_t first,
                                          uint32_t nw8, uint32_t lane) {
    const uint32_t w = first + 8u * lane;
    const uint32_t slot = first & (kRingWords - 1);
    if (w < nw8) {
        const uint8_t *g = words_g + 2u * w;
        dma16(g, lds_addr(ring + slot));
        if (slot == 0 && lane < kMirrorWords / 8) dma16(g, lds_addr(ring + kRingWords));
    }
}

// One decode step of a wave: lane j decodes its next symbol, writes the byte
// to the block's stage at `row` and renormalises from the ring.
template <bool PARTIAL>
__device__ __forceinline__ void stream_step(uint32_t &x, uint32_t &p, const uint2 *T,
                                            const uint16_t *ring, uint8_t *stage_row,
                                            uint32_t lane, bool active) {
    bool need = false;
    if (!PARTIAL || active) {
        const uint2 e = T[x & (kProbScale - 1)];
        x = __umul24(e.x, x >> kProbBits) + e.y;
        stage_row[lane] = (uint8_t)(e.x >> 24);
        need = x < kStateLow;
    }
    const uint64_t mask = __ballot(need);
    if (need) {
        const uint16_t *r = ring + (p & (kRingWords - 1));
        x = (x << 16) | r[lane_prefix(mask)];
    }
    p += (uint32_t)__popcll(mask);
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void decode_stream(
    const SlotEntry *__restrict__ tables, const DevTensor *__restrict__ tensors,
    const DevChunk *__restrict__ chunks, const DevTask *__restrict__ tasks, uint32_t task0,
    const uint8_t *__restrict__ blob, void *__restrict__ out, const float *__restrict__ scales,
    const uint8_t *__restrict__ signmant, int32_t *__restrict__ status) {
    __shared__ uint2 T[kProbScale];
    __shared__ WaveLds<MODE> W[kWaves];

    const DevTask task = tasks[task0 + blockIdx.x];
    const uint32_t kind = tensors[task.tensor].kind;
    const uint32_t cols = tensors[task.tensor].cols;
    load_table(T, tables, task.tensor);

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    const bool has_chunk = wave < task.n_chunks;
    const DevChunk ch = chunks[task.first_chunk + (has_chunk ? wave : 0)];
    const uint8_t *region = blob + ch.byte_offset;
    const uint8_t *words_g = region + kStateBytes;
    WaveLds<MODE> &L = W[wave];
    const uint32_t n = ch.n_symbols;
    const uint32_t nw = ch.n_words;
    const uint32_t nw8 = (nw + 7u) & ~7u;  // the region is padded to 16 bytes

    uint32_t x = has_chunk ? reinterpret_cast<const uint32_t *>(region)[lane] : kStateLow;
    // words issued to the ring / known to have landed
    uint32_t issued = 0, landed = 0;
    if (has_chunk) {
        while (issued < nw && issued < kRingLead) {
            ring_fill(L.ring, words_g, issued, nw8, lane);
            issued += kRingUnit;
        }
        // first block's sign+mantissa bytes (a partial block reads them
        // straight from global memory instead)
        if (MODE == kModeSplit && n >= kBlockSyms && lane < kBlockSyms / 16)
            dma16(signmant + ch.out_elem + 16u * lane, lds_addr(L.sm[0]));
    }
    // vmcnt(0) as a real instruction, so that the compiler also knows the
    // state load has completed and places no wait of its own in the loop
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
    landed = issued;
    __syncthreads();  // table in LDS
    if (!has_chunk) return;

    uint32_t p = 0;
    const uint32_t n_blocks = (n + kBlockSyms - 1) / kBlockSyms;
    const float *scale_row = scales + ch.scale_row;  // the block's row (uniform)
    uint32_t col = ch.col0;  // a multiple of kBlockSyms on this path

    for (uint32_t b = 0; b < n_blocks; ++b) {
        const uint32_t base = b * kBlockSyms;
        const bool full = base + kBlockSyms <= n;
        // ---- ring: the words of this block must have landed; top up ahead
        const uint32_t need_to = (p + kBlockSyms < nw) ? p + kBlockSyms : nw;
        if (landed < need_to) {
            wait_vm1();  // all but the previous block's store
            landed = issued;
        }
        while (issued < nw && issued < p + kRingLead) {
            ring_fill(L.ring, words_g, issued, nw8, lane);
            issued += kRingUnit;
        }
        float scale = 0.f;
        if (MODE == kModeBf16) scale = *scale_row;
        // ---- decode
        if (full) {
#pragma unroll
            for (uint32_t t = 0; t < kBlockSteps; ++t)
                stream_step<false>(x, p, T, L.ring, L.stage + 64u * t, lane, true);
        } else {
            const uint32_t steps = (n - base + 63u) >> 6;
            for (uint32_t t = 0; t < steps; ++t)
                stream_step<true>(x, p, T, L.ring, L.stage + 64u * t, lane,
                                  base + 64u * t + lane < n);
        }
        // ---- output: lane k converts and stores symbols 8k .. 8k+7 of the block
        const uint2 sym8 = *reinterpret_cast<const uint2 *>(L.stage + 8u * lane);
        const uint64_t o = ch.out_elem + base + 8u * lane;
        if (MODE == kModeCodes) {
            if (full) {
                *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(out) + o) = sym8;
            } else {
                const uint8_t *s = reinterpret_cast<const uint8_t *>(&sym8);
                for (uint32_t m = 0; m < 8; ++m)
                    if (base + 8u * lane + m < n) static_cast<uint8_t *>(out)[o + m] = s[m];
            }
        } else {
            uint32_t w[4];
            if (MODE == kModeBf16) {
                float v[8];
                if (kind == ENTQ_SYM_E4M3) {
                    v[0] = __builtin_amdgcn_cvt_f32_fp8((int)sym8.x, 0);
                    v[1] = __builtin_amdgcn_cvt_f32_fp8((int)sym8.x, 1);
                    v[2] = __builtin_amdgcn_cvt_f32_fp8((int)sym8.x, 2);
                    v[3] = __builtin_amdgcn_cvt_f32_fp8((int)sym8.x, 3);
                    v[4] = __builtin_amdgcn_cvt_f32_fp8((int)sym8.y, 0);
                    v[5] = __builtin_amdgcn_cvt_f32_fp8((int)sym8.y, 1);
                    v[6] = __builtin_amdgcn_cvt_f32_fp8((int)sym8.y, 2);
                    v[7] = __builtin_amdgcn_cvt_f32_fp8((int)sym8.y, 3);
                } else {
                    v[0] = (float)((int32_t)(sym8.x << 24) >> 24);
                    v[1] = (float)((int32_t)(sym8.x << 16) >> 24);
                    v[2] = (float)((int32_t)(sym8.x << 8) >> 24);
                    v[3] = (float)((int32_t)sym8.x >> 24);
                    v[4] = (float)((int32_t)(sym8.y << 24) >> 24);
                    v[5] = (float)((int32_t)(sym8.y << 16) >> 24);
                    v[6] = (float)((int32_t)(sym8.y << 8) >> 24);
                    v[7] = (float)((int32_t)sym8.y >> 24);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    w[m] = bf16x2_bits(mul_value_scale(v[2 * m], scale),
                                       mul_value_scale(v[2 * m + 1], scale));
            } else {
                // sign+mantissa bytes of the same 8 elements; rebuild bf16 as
                // sign << 15 | exponent << 7 | mantissa, two per dword
                uint2 sm8;
                if (full) {
                    wait_vm0();
                    sm8 = *reinterpret_cast<const uint2 *>(L.sm[b & 1] + 8u * lane);
                } else {
                    uint8_t sb[8];
                    for (uint32_t m = 0; m < 8; ++m)
                        sb[m] = (base + 8u * lane + m < n) ? signmant[o + m] : 0;
                    sm8 = make_uint2(sb[0] | sb[1] << 8 | sb[2] << 16 | (uint32_t)sb[3] << 24,
                                     sb[4] | sb[5] << 8 | sb[6] << 16 | (uint32_t)sb[7] << 24);
                }
                const uint32_t e4[2] = {sym8.x, sym8.y};
                const uint32_t s4[2] = {sm8.x, sm8.y};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    // bytes (e1 s1 e0 s0) and (e3 s3 e2 s2): each half = e << 8 | s
                    const uint32_t lo = __builtin_amdgcn_perm(e4[h], s4[h], 0x05010400u);
                    const uint32_t hi = __builtin_amdgcn_perm(e4[h], s4[h], 0x07030602u);
                    const uint32_t pr[2] = {lo, hi};
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const uint32_t q = pr[k];
                        // e << 7 from (q >> 1); mantissa from q; sign from q << 8
                        const uint32_t sh = (q >> 1) & 0x7F807F80u;
                        const uint32_t sg = (q << 8) & 0x80008000u;
                        w[2 * h + k] = sh | sg | (q & 0x007F007Fu);
                    }
                }
                // next block's sign+mantissa bytes, if that block is full
                const uint32_t nb = base + kBlockSyms;
                if (nb + kBlockSyms <= n && lane < kBlockSyms / 16)
                    dma16(signmant + ch.out_elem + nb + 16u * lane, lds_addr(L.sm[(b + 1) & 1]));
            }
            uint16_t *o16 = static_cast<uint16_t *>(out) + o;
            if (full) {
                *reinterpret_cast<uint4 *>(o16) = make_uint4(w[0], w[1], w[2], w[3]);
            } else {
                for (uint32_t m = 0; m < 8; ++m)
                    if (base + 8u * lane + m < n) o16[m] = (uint16_t)(w[m >> 1] >> (16 * (m & 1)));
            }
        }
        if (MODE == kModeBf16) {
            col += kBlockSyms;
            if (col == cols) { col = 0; ++scale_row; }
        }
    }
    const uint64_t bad_state = __ballot(x != kStateLow);
    if (status && lane == 0)
        status[ch.status_index] = (p != nw) ? ENTQ_CHUNK_BAD_WORDS
                                  : (bad_state ? ENTQ_CHUNK_BAD_STATE : ENTQ_CHUNK_OK);
    wait_vm0();  // no global->LDS load may outlive the wave (corrupt input stops early)
}

template <int MODE>
int launch_mode(const entq_plan_t *plan, bool stream, int64_t first, int64_t count,
                hipStream_t s, const uint8_t *blob, void *out, const float *scales,
                const uint8_t *signmant, int32_t *status) {
    if (count <= 0) return ENTQ_OK;
    if (first + count > 0x7FFFFFFF) return ENTQ_EINVAL;
    const dim3 grid((unsigned)count), block(kThreads);
    if (stream)
        hipLaunchKernelGGL(decode_stream<MODE>, grid, block, 0, s, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, (uint32_t)first, blob,
                           out, scales, signmant, status);
    else
        hipLaunchKernelGGL(decode_simple<MODE>, grid, block, 0, s, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, (uint32_t)first, blob,
                           out, scales, signmant, status);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

}  // namespace

int launch_decode(const entq_plan_t *plan, int mode, const void *blob, void *out,
                  const float *scales, const uint8_t *signmant, int32_t *status, void *stream) {
    if (plan->n_tasks == 0) return ENTQ_OK;
    hipStream_t s = (hipStream_t)stream;
    const uint8_t *b = static_cast<const uint8_t *>(blob);
    // the streaming kernel takes the tasks it can; the simple one the rest
    const int64_t split = (mode == kModeBf16) ? plan->n_tasks_rows : plan->n_tasks_blocks;
    int r;
    switch (mode) {
    case kModeCodes:
        r = launch_mode<kModeCodes>(plan, true, 0, split, s, b, out, scales, signmant, status);
        if (r == ENTQ_OK)
            r = launch_mode<kModeCodes>(plan, false, split, plan->n_tasks - split, s, b, out,
                                        scales, signmant, status);
        return r;
    case kModeBf16:
        r = launch_mode<kModeBf16>(plan, true, 0, split, s, b, out, scales, signmant, status);
        if (r == ENTQ_OK)
            r = launch_mode<kModeBf16>(plan, false, split, plan->n_tasks - split, s, b, out,
                                       scales, signmant, status);
        return r;
    default:
        r = launch_mode<kModeSplit>(plan, true, 0, split, s, b, out, scales, signmant, status);
        if (r == ENTQ_OK)
            r = launch_mode<kModeSplit>(plan, false, split, plan->n_tasks - split, s, b, out,
                                        scales, signmant, status);
        return r;
    }
}

}  // namespace entq

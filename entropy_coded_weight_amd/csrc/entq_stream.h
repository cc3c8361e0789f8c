// entq_stream.h -- device pieces of the streaming rANS decoder shared by the
// decode kernels and the two fused decode + product kernels: the per-wave
// word ring in LDS fed by direct global->LDS loads, the decode step, the
// fp32 scale / bf16 rounding of decoded Int8 or Float8 codes, the BF16
// merge, and the per-wave staging and priority of the kernels that give each
// wave its own run of chunks. Included by .hip sources only (one private
// copy per translation unit).
#pragma once

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

// The same with a wave-uniform scale taken straight from a scalar register
// (the VOP3 form reads an SGPR as its second operand; no copy to a VGPR).
__device__ __forceinline__ float mul_value_uscale(float v, float s) {
    float r;
    asm("v_mul_f32_e64 %0, %1, %2" : "=v"(r) : "v"(v), "s"(s));
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
// the word ring and the decode step
// ---------------------------------------------------------------------------

// Word ring of one wave: word i of the chunk's stream sits at ring index
// i mod kRingSpan, and the unit at index 0 is also kept at kRingSpan ..
// kRingSpan + kRingUnit - 1 (a mirror), so that the reads of a block -- at
// most kBlockSyms words from a start below kRingSpan -- never wrap: a word's
// LDS address is (ring position + lane offset) * 2, with no mask. The ring is
// refilled in units of kRingUnit words (32 lanes x 16 bytes, one direct
// global->LDS load, two for the unit at index 0) and kept at most kRingLead
// words ahead of the read pointer, which leaves one unit of room for the
// unit in flight. A block reads at most kBlockSyms words, so a unit issued at
// one block's start is not needed before the next block's start.
constexpr uint32_t kRingUnit = 256;
constexpr uint32_t kRingSpan = 3 * kRingUnit;
constexpr uint32_t kRingWords = kRingSpan + kRingUnit;
constexpr uint32_t kRingLead = kRingSpan - kRingUnit;
static_assert(kRingLead >= 2 * kBlockSyms, "a block must find its words loaded a block early");
static_assert(kRingUnit == 32 * 8, "one unit = 32 lanes x 8 words");
static_assert(kRingSpan % kRingUnit == 0 && kBlockSyms <= kRingUnit, "the mirror covers a block");

// One 16-byte global->LDS load per active lane: lane l's bytes land at LDS
// address lds_base + 16 l. The compiler does not see this load, so it inserts
// no wait for it; the kernel waits with explicit vmcnt counts instead.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// All vector-memory operations but the most recent N are complete. The asm
// form is invisible to the compiler's own wait insertion, which therefore
// never relaxes it.
template <int N>
__device__ __forceinline__ void wait_vm() {
    if (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (N == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)p;
}

typedef __attribute__((address_space(3))) const uint16_t lds_u16;

// Uniform bookkeeping of one chunk on the streaming path. The steps advance
// only pos; the stream index of the next word is base + pos - ring / 2.
struct Stream {
    const uint8_t *words_g;     // the chunk's word stream in global memory
    uint32_t ring;              // LDS byte address of the wave's ring
    uint32_t pos;               // LDS address / 2 of the next word to read
    uint32_t base;              // stream index of the word at ring index 0
    uint32_t nw, nw8;           // words, and words rounded up to 8 (16 bytes)
    uint32_t issued, landed;    // words loaded into the ring / known landed
    uint32_t hpos;              // ring_service is due once pos passes this
};

// Words consumed so far.
__device__ __forceinline__ uint32_t ring_consumed(const Stream &s) {
    return s.base + s.pos - (s.ring >> 1);
}

// Loads words [issued, issued + kRingUnit) of the chunk into the ring (lanes
// whose 16 bytes lie inside the chunk's region).
__device__ __forceinline__ void ring_fill(const Stream &s, uint32_t lane) {
    const uint32_t w = s.issued + 8u * lane;
    const uint32_t at = s.issued % kRingSpan;
    if (lane < kRingUnit / 8 && w < s.nw8) {
        dma16(s.words_g + 2u * w, s.ring + 2u * at);
        if (at == 0) dma16(s.words_g + 2u * w, s.ring + 2u * kRingSpan);  // the mirror
    }
}

// The next point at which a block start needs ring_service: once a block
// could read past the landed words, or the ring could take another unit, or
// the read position reaches the end of the span (a block must start below it).
__device__ __forceinline__ void ring_horizon(Stream &s) {
    const uint32_t a = (s.landed >= s.nw) ? 0xFFFFFFFFu : s.landed - kBlockSyms;
    const uint32_t b = (s.issued >= s.nw) ? 0xFFFFFFFFu : s.issued - kRingLead;
    const uint32_t h = (a < b ? a : b) - s.base;  // both are at or past the consumed words
    s.hpos = (s.ring >> 1) + (h < kRingSpan ? h : kRingSpan - 1);
}

// Chunk start: the stream of a region's words, its first units in flight.
// The caller waits for them (vmcnt(0)) and then calls ring_horizon.
__device__ __forceinline__ void ring_open(Stream &s, const uint8_t *words_g, uint32_t ring,
                                          uint32_t n_words, uint32_t lane) {
    s.words_g = words_g;
    s.ring = ring;
    s.pos = ring >> 1;
    s.base = 0;
    s.nw = n_words;
    s.nw8 = (n_words + 7u) & ~7u;  // the region is padded to 16 bytes
    s.issued = 0;
    while (s.issued < s.nw && s.issued < kRingLead) {
        ring_fill(s, lane);
        s.issued += kRingUnit;
    }
}

// Block start, slow path: moves the read position back below the span,
// makes sure this block's words have landed, tops the ring up to kRingLead
// words ahead and sets the next horizon.
__device__ __forceinline__ void ring_service(Stream &s, uint32_t lane) {
    if (s.pos - (s.ring >> 1) >= kRingSpan) {
        s.pos -= kRingSpan;
        s.base += kRingSpan;
    }
    const uint32_t p = ring_consumed(s);
    const uint32_t need_to = (p + kBlockSyms < s.nw) ? p + kBlockSyms : s.nw;
    if (s.landed < need_to) {
        wait_vm<1>();  // everything but the previous block's store
        s.landed = s.issued;
    }
    while (s.issued < s.nw && s.issued < p + kRingLead) {
        ring_fill(s, lane);
        s.issued += kRingUnit;
    }
    ring_horizon(s);
}

// One decode step of a wave: lane j decodes its next symbol (stores the
// high half of its table entry in the stage) and renormalises from the
// ring. Every lane reads the ring (no branch on the mask; a lane that does
// not renormalise reads a word at or before the step's last one); lanes
// that renormalise shift the word in, the others keep x (v_perm with a
// per-lane selector). pos is the ring position of the step's first word;
// within a block it stays below kRingSpan + kBlockSyms, inside the mirror.
template <bool PARTIAL>
__device__ __forceinline__ void stream_step(uint32_t &x, uint32_t &pos, const uint2 *T,
                                            uint16_t *stage_row, uint32_t lane, bool active) {
    bool need = false;
    if (!PARTIAL || active) {
        const uint2 e = T[x & (kProbScale - 1)];
        x = __umul24(e.x, x >> kProbBits) + e.y;
        stage_row[lane] = (uint16_t)(e.x >> 16);
        need = x < kStateLow;
    }
    const uint64_t mask = __ballot(need);
    const uint32_t w = *reinterpret_cast<lds_u16 *>((pos + lane_prefix(mask)) << 1);
    x = __builtin_amdgcn_perm(x, w, need ? 0x05040100u : 0x07060504u);
    pos += (uint32_t)__popcll(mask);
}

// The value of an e4m3 NaN code (S.1111.111) is the NaN that keeps the
// code's sign and puts its mantissa bits at the top of the fp32 payload:
// S << 31 | 0x7FF00000 (a NaN widened into a wider format, IEEE 754-2008
// §6.2.3). The conversion instruction returns one fixed NaN for both codes,
// so the NaN codes are patched. Element-wise form, code in bits 0..7:
__device__ __forceinline__ float e4m3_value(uint32_t code) {
    const float v = __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
    return ((code & 0x7Fu) == 0x7Fu) ? __uint_as_float(((code & 0x80u) << 24) | 0x7FF00000u) : v;
}

// Two bf16 results r of the codes in bytes 1 and 3 of d: the half whose
// code is a NaN code becomes that NaN's bf16, S << 15 | 0x7FF0, whatever
// the scale (the code's NaN wins over a NaN scale, and a NaN stays a NaN
// through the product and the rounding).
__device__ __forceinline__ uint32_t e4m3_nan_patch2(uint32_t d, uint32_t r) {
    // bit 15 / 31 set iff the code's low 7 bits are all ones
    const uint32_t hit = ((d & 0x7F007F00u) + 0x01000100u) & 0x80008000u;
    const uint32_t sel = (hit >> 15) * 0xFFFFu;
    return (r & ~sel) | (((d & 0x80008000u) | 0x7FF07FF0u) & sel);
}

// bf16 of (value of a code byte) * scale, two per dword; d holds two staged
// 16-bit slots, the code bytes in bytes 1 and 3.
template <bool E4M3>
__device__ __forceinline__ uint32_t dequant2(uint32_t d, float scale) {
    float v0, v1;
    if (E4M3) {
        v0 = __builtin_amdgcn_cvt_f32_fp8((int)d, 1);
        v1 = __builtin_amdgcn_cvt_f32_fp8((int)d, 3);
    } else {
        v0 = (float)((int32_t)(d << 16) >> 24);
        v1 = (float)((int32_t)d >> 24);
    }
    const uint32_t r = bf16x2_bits(mul_value_uscale(v0, scale), mul_value_uscale(v1, scale));
    return E4M3 ? e4m3_nan_patch2(d, r) : r;
}

// sign << 15 | exponent << 7 | mantissa for two elements: q holds, per
// 16-bit half, exponent << 8 | sign+mantissa byte.
__device__ __forceinline__ uint32_t merge2(uint32_t q) {
    return ((q >> 1) & 0x7F807F80u) | ((q << 8) & 0x80008000u) | (q & 0x007F007Fu);
}

// ---------------------------------------------------------------------------
// pieces of the kernels that give each wave its own run of chunks
// ---------------------------------------------------------------------------

// Per-wave staging: a decoded step stores, per lane, the high half of its
// slot-table entry (symbol << 8), so the symbol is byte 1 of a 16-bit slot.
struct alignas(16) WaveStage {
    uint16_t stage[kBlockSyms];
};

// Split mode: blocks of sign+mantissa bytes in flight per wave.
constexpr uint32_t kSmAhead = 4;

// Sign+mantissa bytes that lane k merges into its 4 outputs (columns) of a
// block.
__device__ __forceinline__ uint32_t load_sm4(const uint8_t *sm_block, uint32_t lane) {
    return *reinterpret_cast<const uint32_t *>(sm_block + 4u * lane);
}

// Progress-based wave priority: a wave drops one level once it has done
// half of its blocks, again at three quarters and at seven eighths (half of
// what is left each time), so waves that are behind win issue arbitration
// near the end. (The default favours the oldest waves: the younger
// workgroup on a CU, and the younger waves of a workgroup, then finish long
// after the rest, with the CU half idle. Drops every quarter of the blocks,
// or from the first eighth on, left a longer tail.)
struct Prio {
    uint32_t my_blocks, done, at, level;
    __device__ __forceinline__ void start(uint32_t blocks) {
        my_blocks = blocks;
        done = 0;
        at = blocks / 2 ? blocks / 2 : 1;
        level = 3;
        __builtin_amdgcn_s_setprio(3);
    }
    __device__ __forceinline__ void tick() {
        if (__builtin_expect(++done == at, 0)) {
            at += (my_blocks - at) / 2 ? (my_blocks - at) / 2 : 1;
            --level;
            if (level == 2) __builtin_amdgcn_s_setprio(2);
            else if (level == 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        }
    }
};

}  // namespace
}  // namespace entq

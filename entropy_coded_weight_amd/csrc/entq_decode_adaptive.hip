// entq_decode_adaptive.hip -- gfx950 decode of chunks that carry their own
// frequency tables.
//
// EntroLLM names adaptive entropy coding as its next step [EntroLLM summary,
// "Significado y Afirmaciones"]. Here every chunk is coded with the table of
// its own symbol counts, stored at the head of its region (u16 freq[256]),
// so a chunk follows its local statistics instead of its tensor's.
//
// Mapping onto CDNA4. The shared-table decoder keeps one 32 KB slot table
// per workgroup; with a table per chunk every wave needs its own, so the
// slot table is split into a 4 KB slot -> symbol map and a 1 KB symbol ->
// (f, cum) map, built by the wave from its chunk's 512-byte header before it
// decodes the chunk: a wave scan of the frequencies gives the cumulative
// starts, then each lane fills 64 consecutive slots (a binary search for the
// symbol of its first slot, then a walk). A decode step reads both maps (two
// dependent LDS reads instead of one); the word ring, the staged 4-step
// blocks and the fused scale/bf16 store are the streaming decoder's
// (entq_stream.h). Waves share nothing, so no workgroup barrier is needed;
// wave g of the grid decodes chunks g, g + G, g + 2G, ...
#include <hip/hip_runtime.h>

#include <algorithm>

#include "entq.h"
#include "entq_internal.h"
#include "entq_stream.h"

namespace entq {
namespace {

constexpr int kAdWaves = 7;  // 7.5 KB of LDS each: three workgroups per CU
constexpr int kAdThreads = kAdWaves * 64;

struct alignas(16) AdaptiveWave {
    uint8_t sym[kProbScale];     // slot -> symbol
    uint32_t ent[256];           // symbol -> f | cum << 16
    uint16_t stage[kBlockSyms];  // one block of staged symbols (symbol << 8)
};

// One decode step with the chunk's own maps; otherwise as stream_step.
template <bool PARTIAL>
__device__ __forceinline__ void adaptive_step(uint32_t &x, uint32_t &pos, const uint8_t *SYM,
                                              const uint32_t *ENT, uint16_t *stage_row,
                                              uint32_t lane, bool active) {
    bool need = false;
    if (!PARTIAL || active) {
        const uint32_t slot = x & (kProbScale - 1);
        const uint32_t s = SYM[slot];
        const uint32_t e = ENT[s];
        x = __umul24(e & 0x1FFFu, x >> kProbBits) + slot - (e >> 16);
        stage_row[lane] = (uint16_t)(s << 8);
        need = x < kStateLow;
    }
    const uint64_t mask = __ballot(need);
    const uint32_t w = *reinterpret_cast<lds_u16 *>((pos + lane_prefix(mask)) << 1);
    x = __builtin_amdgcn_perm(x, w, need ? 0x05040100u : 0x07060504u);
    pos += (uint32_t)__popcll(mask);
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Builds the wave's maps from a chunk's table; false if it does not sum to
// 4096.
__device__ __forceinline__ bool build_maps(const uint8_t *table, AdaptiveWave &W, uint32_t lane) {
    const uint2 fr = *reinterpret_cast<const uint2 *>(table + 8u * lane);  // entries 4l .. 4l+3
    const uint32_t f0 = fr.x & 0xFFFFu, f1 = fr.x >> 16, f2 = fr.y & 0xFFFFu, f3 = fr.y >> 16;
    const uint32_t own = f0 + f1 + f2 + f3;
    uint32_t incl = own;  // inclusive scan over the lanes
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint32_t v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    const uint32_t total = __shfl(incl, 63);
    if (total != kProbScale) return false;
    const uint32_t c0 = incl - own;
    W.ent[4u * lane + 0] = f0 | (c0 << 16);
    W.ent[4u * lane + 1] = f1 | ((c0 + f0) << 16);
    W.ent[4u * lane + 2] = f2 | ((c0 + f0 + f1) << 16);
    W.ent[4u * lane + 3] = f3 | ((c0 + f0 + f1 + f2) << 16);
    wave_sync();
    // lane l fills slots 64 l .. 64 l + 63: the symbol of a slot is the last
    // one whose cumulative start is at or below it
    const uint32_t j0 = 64u * lane;
    uint32_t s = 0;
#pragma unroll
    for (uint32_t step = 128; step; step >>= 1)
        if ((W.ent[s + step] >> 16) <= j0) s += step;  // s + step <= 255
    uint32_t next = s < 255 ? (W.ent[s + 1] >> 16) : kProbScale;
    for (uint32_t k = 0; k < 64; k += 4) {
        uint32_t packed = 0;
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
            const uint32_t j = j0 + k + q;
            while (next <= j) {
                ++s;
                next = s < 255 ? (W.ent[s + 1] >> 16) : kProbScale;
            }
            packed |= s << (8 * q);
        }
        *reinterpret_cast<uint32_t *>(W.sym + j0 + k) = packed;
    }
    wave_sync();
    return true;
}

template <int MODE>
__global__ __launch_bounds__(kAdThreads) void decode_adaptive(
    const DevTensor *__restrict__ tensors, const DevChunk *__restrict__ chunks, uint32_t n_chunks,
    const uint8_t *__restrict__ blob, void *__restrict__ out, const float *__restrict__ scales,
    const uint8_t *__restrict__ signmant, int32_t *__restrict__ status) {
    __shared__ __attribute__((aligned(16))) uint16_t RING[kAdWaves][kRingWords];
    __shared__ AdaptiveWave WV[kAdWaves];

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    AdaptiveWave &W = WV[wave];
    const uint32_t waves = gridDim.x * kAdWaves;
    for (uint32_t c = blockIdx.x * kAdWaves + wave; c < n_chunks; c += waves) {
        const DevChunk ch = chunks[c];
        const DevTensor td = tensors[ch.tensor];
        const uint8_t *region = blob + ch.byte_offset;
        if (!build_maps(region, W, lane)) {
            if (status && lane == 0) status[ch.status_index] = ENTQ_CHUNK_BAD_TABLE;
            continue;
        }
        const uint8_t *body = region + ENTQ_TABLE_BYTES;
        const uint32_t n = ch.n_symbols;
        uint32_t x = reinterpret_cast<const uint32_t *>(body)[lane];
        Stream s;
        ring_open(s, body + kStateBytes, lds_addr(RING[wave]), ch.n_words, lane);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): states and the first ring units
        s.landed = s.issued;
        ring_horizon(s);
        const bool e4m3 = td.kind == ENTQ_SYM_E4M3;
        const uint32_t cols = td.cols;
        const float *scale_row = scales + ch.scale_row;
        float scale = (MODE == kModeBf16) ? *scale_row : 0.f;
        uint32_t col = ch.col0;  // a multiple of kBlockSyms
        uint16_t *o16 = static_cast<uint16_t *>(out) + ch.out_elem;
        uint8_t *o8 = static_cast<uint8_t *>(out) + ch.out_elem;
        // sign+mantissa bytes of the chunk's elements (split mode)
        const uint8_t *sm_g = (MODE == kModeSplit) ? signmant + ch.out_elem : nullptr;
        const uint32_t full_blocks = n / kBlockSyms;
        for (uint32_t b = 0; b < full_blocks; ++b) {
            if (__builtin_expect(s.pos > s.hpos, 0)) ring_service(s, lane);
            // this lane's four sign+mantissa bytes of the block, in flight
            // while the block decodes
            uint32_t sm4 = 0;
            if (MODE == kModeSplit) sm4 = *reinterpret_cast<const uint32_t *>(sm_g + 4u * lane);
#pragma unroll
            for (uint32_t t = 0; t < kBlockSteps; ++t)
                adaptive_step<false>(x, s.pos, W.sym, W.ent, W.stage + 64u * t, lane, true);
            const uint2 d = *reinterpret_cast<const uint2 *>(W.stage + 4u * lane);
            if (MODE == kModeCodes) {
                reinterpret_cast<uint32_t *>(o8)[lane] = __builtin_amdgcn_perm(d.y, d.x, 0x07050301u);
                o8 += kBlockSyms;
            } else if (MODE == kModeSplit) {
                // per 16-bit half: exponent << 8 | sign+mantissa
                const uint2 w = make_uint2(merge2(__builtin_amdgcn_perm(d.x, sm4, 0x07010500u)),
                                           merge2(__builtin_amdgcn_perm(d.y, sm4, 0x07030502u)));
                reinterpret_cast<uint2 *>(o16)[lane] = w;
                o16 += kBlockSyms;
                sm_g += kBlockSyms;
            } else {
                if (col == cols) {
                    col = 0;
                    ++scale_row;
                    scale = *scale_row;
                }
                const uint2 w = e4m3 ? make_uint2(dequant2<true>(d.x, scale), dequant2<true>(d.y, scale))
                                     : make_uint2(dequant2<false>(d.x, scale), dequant2<false>(d.y, scale));
                reinterpret_cast<uint2 *>(o16)[lane] = w;
                o16 += kBlockSyms;
                col += kBlockSyms;
            }
        }
        // the last, partial block (a tensor's last chunk): element-wise output
        const uint32_t rest = n - full_blocks * kBlockSyms;
        if (rest) {
            if (s.pos > s.hpos) ring_service(s, lane);
            if (MODE == kModeBf16 && col == cols) {
                ++scale_row;
                scale = *scale_row;
            }
            for (uint32_t t = 0; 64u * t < rest; ++t)
                adaptive_step<true>(x, s.pos, W.sym, W.ent, W.stage + 64u * t, lane,
                                    64u * t + lane < rest);
            const uint2 d = *reinterpret_cast<const uint2 *>(W.stage + 4u * lane);
            const uint32_t sym4 = __builtin_amdgcn_perm(d.y, d.x, 0x07050301u);
            for (uint32_t m = 0; m < 4; ++m) {
                const uint32_t i = 4u * lane + m;
                if (i >= rest) break;
                const uint32_t sym = (sym4 >> (8 * m)) & 0xFFu;
                if (MODE == kModeCodes) {
                    o8[i] = (uint8_t)sym;
                } else if (MODE == kModeSplit) {
                    const uint32_t sm = sm_g[i];
                    o16[i] = (uint16_t)(((sm & 0x80u) << 8) | (sym << 7) | (sm & 0x7Fu));
                } else {
                    const float v = e4m3 ? __builtin_amdgcn_cvt_f32_fp8((int)sym, 0)
                                         : (float)(int8_t)sym;
                    o16[i] = bf16_bits(mul_value_scale(v, scale));
                }
            }
        }
        const uint64_t bad_state = __ballot(x != kStateLow);
        if (status && lane == 0)
            status[ch.status_index] = (ring_consumed(s) != s.nw) ? ENTQ_CHUNK_BAD_WORDS
                                      : (bad_state ? ENTQ_CHUNK_BAD_STATE : ENTQ_CHUNK_OK);
        wait_vm<0>();  // no global->LDS load may outlive the chunk
        wave_sync();   // the maps are rebuilt for the next chunk
    }
}

}  // namespace

int launch_decode_adaptive(const entq_plan_t *plan, int mode, const void *blob, void *out,
                           const float *scales, const uint8_t *signmant, int32_t *status,
                           void *stream) {
    if (plan->n_chunks == 0) return ENTQ_OK;
    if (plan->n_chunks > 0xFFFFFFFFll) return ENTQ_EINVAL;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return ENTQ_EHIP;
    const void *k = (mode == kModeBf16)    ? (const void *)decode_adaptive<kModeBf16>
                    : (mode == kModeSplit) ? (const void *)decode_adaptive<kModeSplit>
                                           : (const void *)decode_adaptive<kModeCodes>;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kAdThreads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const int64_t need = (plan->n_chunks + kAdWaves - 1) / kAdWaves;
    const int64_t grid = std::min<int64_t>(need, (int64_t)cus * per_cu);
    const uint32_t nc = (uint32_t)plan->n_chunks;
    const uint8_t *b = static_cast<const uint8_t *>(blob);
    const dim3 g((unsigned)grid), blk(kAdThreads);
    const hipStream_t st = (hipStream_t)stream;
    if (mode == kModeBf16)
        hipLaunchKernelGGL(decode_adaptive<kModeBf16>, g, blk, 0, st, plan->d_tensors,
                           plan->d_chunks, nc, b, out, scales, signmant, status);
    else if (mode == kModeSplit)
        hipLaunchKernelGGL(decode_adaptive<kModeSplit>, g, blk, 0, st, plan->d_tensors,
                           plan->d_chunks, nc, b, out, scales, signmant, status);
    else
        hipLaunchKernelGGL(decode_adaptive<kModeCodes>, g, blk, 0, st, plan->d_tensors,
                           plan->d_chunks, nc, b, out, scales, signmant, status);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

}  // namespace entq

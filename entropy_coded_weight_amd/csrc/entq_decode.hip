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
//    LDS for a block of 4 steps and leave as 4 consecutive outputs per lane
//    (one 8-byte store for bf16), the fp32 row-scale multiply and the bf16
//    rounding fused into that store. Like DFloat11's kernel it stages output
//    on chip and writes it coalesced [DFloat11 write-up, "Kernels GPU de 2
//    etapas y metadatos auxiliares"], but rANS needs no counting pass: a
//    chunk's output position is known up front.
//  * decode_simple: one symbol per lane per step straight from global
//    memory; used for tensors whose chunk size or row length is not a
//    multiple of the 256-symbol block.
#include <hip/hip_runtime.h>

#include <atomic>

#include "entq.h"
#include "entq_internal.h"
#include "entq_stream.h"

namespace entq {
namespace {

// ---------------------------------------------------------------------------
// decode_simple
// ---------------------------------------------------------------------------

template <int MODE>
__device__ __forceinline__ void simple_chunk(const uint2 *T, const DevTensor &td, const DevChunk &ch,
                                             const uint8_t *__restrict__ blob, void *__restrict__ out,
                                             const float *__restrict__ scales,
                                             const uint8_t *__restrict__ signmant,
                                             int32_t *__restrict__ status, uint32_t lane) {
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
                                    ? e4m3_value(sym)
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
    for (uint32_t c = wave; c < task.n_chunks; c += kWaves)
        simple_chunk<MODE>(T, td, chunks[task.first_chunk + c], blob, out, scales, signmant,
                           status, lane);
}

// ---------------------------------------------------------------------------
// decode_stream
// ---------------------------------------------------------------------------

// The full blocks of one chunk to bf16. The e4m3 / int8 choice is made once
// per chunk (a template argument), and rows are counted down in blocks: the
// next row's scale is loaded once the last block of a row is converted, if
// that row has a block in this chunk (no scale past the chunk's last row is
// read). (Moving a block's conversion and store into the LDS-read shadows of
// the next block's first step made the layer decode 15 % slower.)
template <bool E4M3, bool PRIO>
__device__ __forceinline__ void blocks_bf16(Stream &s, uint32_t &x, const uint2 *T,
                                            uint16_t *stage, uint32_t lane, uint32_t full_blocks,
                                            uint32_t cols, uint32_t &col,
                                            const float *&scale_row, float &scale,
                                            uint16_t *&o16, Prio &pr) {
    // blocks of the current row still to convert (col is a multiple of the block)
    uint32_t row_left = (cols - col) / kBlockSyms;
    const uint32_t row_blocks = cols / kBlockSyms;
    for (uint32_t b = 0; b < full_blocks; ++b) {
        if (PRIO) pr.tick();
        if (__builtin_expect(s.pos > s.hpos, 0)) ring_service(s, lane);
#pragma unroll
        for (uint32_t t = 0; t < kBlockSteps; ++t)
            stream_step<false>(x, s.pos, T, stage + 64u * t, lane, true);
        // lane k: symbols 4k .. 4k+3 of the block (bytes 1, 3, 5, 7)
        const uint2 d = *reinterpret_cast<const uint2 *>(stage + 4u * lane);
        reinterpret_cast<uint2 *>(o16)[lane] =
            make_uint2(dequant2<E4M3>(d.x, scale), dequant2<E4M3>(d.y, scale));
        o16 += kBlockSyms;
        if (__builtin_expect(--row_left == 0, 0) && b + 1 < full_blocks) {  // b ends a row
            row_left = row_blocks;
            ++scale_row;
            scale = *scale_row;
        }
    }
    col = cols - row_left * kBlockSyms;
}

// PRIO: progress-based wave priority (Prio); off for launches with one
// chunk per workgroup, where the waves do not compete and its per-block
// bookkeeping only lengthens each wave's chain.
template <int MODE, bool PRIO>
__global__ __launch_bounds__(kThreads) ENTQ_TWO_WORKGROUPS_SGPRS void decode_stream(
    const SlotEntry *__restrict__ tables, const DevTensor *__restrict__ tensors,
    const DevChunk *__restrict__ chunks, const DevTask *__restrict__ tasks, uint32_t task0,
    const uint8_t *__restrict__ blob, void *__restrict__ out, const float *__restrict__ scales,
    const uint8_t *__restrict__ signmant, int32_t *__restrict__ status) {
    __shared__ __attribute__((aligned(16))) uint16_t RING[kWaves][kRingWords];
    __shared__ uint2 T[kProbScale];
    __shared__ WaveStage STG[kWaves];

    const DevTask task = tasks[task0 + blockIdx.x];
    const bool e4m3 = tensors[task.tensor].kind == ENTQ_SYM_E4M3;
    const uint32_t cols = tensors[task.tensor].cols;
    load_table(T, tables, task.tensor);
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    WaveStage &G = STG[wave];
    // the task's chunks in rounds: every round keeps the same number of waves
    // busy, except that a run of two or more rounds that 14 waves finish in as
    // many rounds goes to 14 waves (on runs of 25-26 chunks, 14 busy waves
    // decode 0.4 % faster than two equal rounds of 13; 15 or 16 are slower)
    const uint32_t rounds = (task.n_chunks + kWaves - 1) / kWaves;
    const uint32_t even = (task.n_chunks + rounds - 1) / rounds;
    const uint32_t width = (rounds > 1 && (task.n_chunks + 13) / 14 == rounds && even < 14) ? 14u
                                                                                          : even;
    // progress-based priority, restarted for each chunk: a wave starts each
    // of its chunks at the top level and drops at a half, three quarters and
    // seven eighths of that chunk's blocks (one countdown over the wave's
    // whole run of chunks was 1 % slower)
    Prio pr = {};
    for (uint32_t c = wave; wave < width && c < task.n_chunks; c += width) {
        const DevChunk ch = chunks[task.first_chunk + c];
        if (PRIO) pr.start(ch.n_symbols / kBlockSyms);
        const uint8_t *region = blob + ch.byte_offset;
        const uint32_t n = ch.n_symbols;
        uint32_t x = reinterpret_cast<const uint32_t *>(region)[lane];
        Stream s;
        ring_open(s, region + kStateBytes, lds_addr(RING[wave]), ch.n_words, lane);
        const uint8_t *sm_g = signmant + ch.out_elem;
        const uint32_t full_blocks = n / kBlockSyms;
        // split mode: the sign+mantissa bytes of block b are loaded into
        // register smr[b % kSmAhead] kSmAhead blocks ahead of their use (the
        // block loop is unrolled kSmAhead times, so the registers are never
        // copied: a copy would wait for the load in flight)
        uint32_t smr[kSmAhead] = {};
        if (MODE == kModeSplit)
#pragma unroll
            for (uint32_t j = 0; j < kSmAhead; ++j)
                if (j < full_blocks) smr[j] = load_sm4(sm_g + j * kBlockSyms, lane);
        // vmcnt(0) as a real instruction, so that the compiler also knows the
        // state load has completed and places no wait of its own in the loop
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) expcnt(7) lgkmcnt(15)
        s.landed = s.issued;
        ring_horizon(s);
        const float *scale_row = scales + ch.scale_row;
        float scale = (MODE == kModeBf16) ? *scale_row : 0.f;
        uint32_t col = ch.col0;  // a multiple of kBlockSyms on this path
        uint16_t *o16 = static_cast<uint16_t *>(out) + ch.out_elem;
        uint8_t *o8 = static_cast<uint8_t *>(out) + ch.out_elem;

        auto block = [&](uint32_t b, uint32_t &sm_reg) __attribute__((always_inline)) {
            if (PRIO) pr.tick();
            if (__builtin_expect(s.pos > s.hpos, 0)) ring_service(s, lane);
#pragma unroll
            for (uint32_t t = 0; t < kBlockSteps; ++t)
                stream_step<false>(x, s.pos, T, G.stage + 64u * t, lane, true);
            // lane k: symbols 4k .. 4k+3 of the block (bytes 1, 3, 5, 7)
            const uint2 d = *reinterpret_cast<const uint2 *>(G.stage + 4u * lane);
            if (MODE == kModeCodes) {
                reinterpret_cast<uint32_t *>(o8)[lane] = __builtin_amdgcn_perm(d.y, d.x, 0x07050301u);
                o8 += kBlockSyms;
            } else {
                // per 16-bit half: exponent << 8 | sign+mantissa
                const uint2 w = make_uint2(merge2(__builtin_amdgcn_perm(d.x, sm_reg, 0x07010500u)),
                                           merge2(__builtin_amdgcn_perm(d.y, sm_reg, 0x07030502u)));
                // block b + kSmAhead's bytes into the register just consumed
                // (past the last full block: this block's again, unused). The
                // load is unconditional and kept after the merge, so that the
                // register is reused in place: a copy would wait for it.
                __builtin_amdgcn_sched_barrier(0);
                sm_reg = load_sm4(sm_g + (b + kSmAhead < full_blocks ? kSmAhead * kBlockSyms : 0u),
                                  lane);
                sm_g += kBlockSyms;
                reinterpret_cast<uint2 *>(o16)[lane] = w;
                o16 += kBlockSyms;
            }
        };
        uint32_t b = 0;
        if (MODE == kModeBf16) {
            if (e4m3)
                blocks_bf16<true, PRIO>(s, x, T, G.stage, lane, full_blocks, cols, col, scale_row,
                                        scale, o16, pr);
            else
                blocks_bf16<false, PRIO>(s, x, T, G.stage, lane, full_blocks, cols, col,
                                         scale_row, scale, o16, pr);
        } else if (MODE == kModeSplit) {
            for (; b + kSmAhead <= full_blocks; b += kSmAhead)
#pragma unroll
                for (uint32_t j = 0; j < kSmAhead; ++j) block(b + j, smr[j]);
#pragma unroll
            for (uint32_t j = 0; j < kSmAhead; ++j)
                if (b + j < full_blocks) block(b + j, smr[j]);
        } else {
            for (; b < full_blocks; ++b) block(b, smr[0]);
        }
        // the last, partial block: one symbol per lane and step, element-wise output
        const uint32_t rest = n - full_blocks * kBlockSyms;
        if (rest) {
            if (s.pos > s.hpos) ring_service(s, lane);
            if (MODE == kModeBf16 && col == cols) {
                ++scale_row;
                scale = *scale_row;
            }
            for (uint32_t t = 0; 64u * t < rest; ++t)
                stream_step<true>(x, s.pos, T, G.stage + 64u * t, lane, 64u * t + lane < rest);
            const uint2 d = *reinterpret_cast<const uint2 *>(G.stage + 4u * lane);
            const uint32_t sym4 = __builtin_amdgcn_perm(d.y, d.x, 0x07050301u);
            for (uint32_t m = 0; m < 4; ++m) {
                const uint32_t i = 4u * lane + m;
                if (i >= rest) break;
                const uint32_t sym = (sym4 >> (8 * m)) & 0xFFu;
                if (MODE == kModeCodes) {
                    o8[i] = (uint8_t)sym;
                } else if (MODE == kModeBf16) {
                    const float v = e4m3 ? e4m3_value(sym)
                                         : (float)(int8_t)sym;
                    o16[i] = bf16_bits(mul_value_scale(v, scale));
                } else {
                    const uint32_t sm = sm_g[i];
                    o16[i] = (uint16_t)(((sm & 0x80u) << 8) | (sym << 7) | (sm & 0x7Fu));
                }
            }
        }
        const uint64_t bad_state = __ballot(x != kStateLow);
        if (status && lane == 0)
            status[ch.status_index] = (ring_consumed(s) != s.nw) ? ENTQ_CHUNK_BAD_WORDS
                                      : (bad_state ? ENTQ_CHUNK_BAD_STATE : ENTQ_CHUNK_OK);
        wait_vm<0>();  // no global->LDS load may outlive the chunk (corrupt input stops early)
    }
}

template <int MODE>
__host__ int64_t stream_occupancy() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_stream<MODE, true>, kThreads, 0) !=
        hipSuccess)
        return 0;
    return blocks;
}

template <int MODE>
int launch_mode(const entq_plan_t *plan, bool stream, int64_t first, int64_t count,
                hipStream_t s, const uint8_t *blob, void *out, const float *scales,
                const uint8_t *signmant, int32_t *status) {
    if (count <= 0) return ENTQ_OK;
    if (first + count > 0x7FFFFFFF) return ENTQ_EINVAL;
    const dim3 grid((unsigned)count), block(kThreads);
    const bool prio = (MODE == kModeBf16 ? plan->max_task_chunks_rows
                                         : plan->max_task_chunks_blocks) > 1;
    if (stream && prio)
        hipLaunchKernelGGL((decode_stream<MODE, true>), grid, block, 0, s, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, (uint32_t)first, blob,
                           out, scales, signmant, status);
    else if (stream)
        hipLaunchKernelGGL((decode_stream<MODE, false>), grid, block, 0, s, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, (uint32_t)first, blob,
                           out, scales, signmant, status);
    else
        hipLaunchKernelGGL(decode_simple<MODE>, grid, block, 0, s, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, (uint32_t)first, blob,
                           out, scales, signmant, status);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

}  // namespace

int64_t resident_workgroups() {
    // per device, computed once (threads that race here store the same value)
    static std::atomic<int64_t> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int64_t v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        int64_t per_cu = stream_occupancy<kModeSplit>();  // the largest LDS footprint
        if (per_cu <= 0) per_cu = 1;
        v = (int64_t)cus * per_cu;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

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

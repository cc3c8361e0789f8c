// entq_decode_gemv.hip -- gfx950 kernel of the fused decode + product for a
// few activation rows, on the vector units inside the decode loop.
//
// Y[i][r] = sum_c X[i][c] * bf16(W)[r][c] for m <= kGemvMaxRows rows of X,
// bf16(W) exactly as the bf16 decode writes it. With so few activation rows
// the product needs no matrix cores: after a block's 4 steps each lane holds
// 4 consecutive weights of one weight row as two bf16 pairs, and adds their
// products with the same 4 columns of every activation row into fp32 sums
// (v_dot2_f32_bf16: two products and their sum in one instruction). At the
// end of a weight row the 64 lanes' sums are added in a fixed tree and one
// lane writes the results. The waves work as in decode_stream -- each on its
// own chunks, with no barrier and no lockstep; word ring, slot table and
// priority unchanged -- and the block's store is replaced by the products,
// so chunks may hold several rows. This is the decode phase of inference at
// batch 1 to 4, where the weights are needed once per generated token
// [EntQuant, "Float8@2bits: Entropy Coding Enables Data-Free Model
// Compression", technical summary §2 "Decodificación en Tiempo de
// Inferencia"].
#include <hip/hip_runtime.h>

#include "entq.h"
#include "entq_internal.h"
#include "entq_stream.h"

namespace entq {
namespace {

struct GemvTensor {
    const uint16_t *x;  // bf16 activations: m rows, row stride ldx elements
    float *y;           // fp32 results: m rows, row stride ldy
    uint64_t ldx, ldy;
    uint64_t row0;      // scale row of the tensor's weight row 0
};
struct GemvArgs {
    GemvTensor t[kGemvMaxTensors];
    uint32_t m;
};

__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t a, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, a), acc, false);
}

// The sum of v over the wave's 64 lanes: a butterfly whose every level adds
// the same two values on both partner lanes, so all lanes end with the same
// bits, and the order is fixed.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// One chunk (whole rows) of a decode_gemv task.
template <int M, bool E4M3, bool SPLIT, bool PRIO>
__device__ __forceinline__ void gemv_chunk(const DevChunk &ch, const uint8_t *__restrict__ blob,
                                           const uint2 *T, uint16_t *ring_lds, uint16_t *stage,
                                           uint32_t lane, uint32_t cols,
                                           const float *__restrict__ scales,
                                           const uint8_t *__restrict__ signmant,
                                           const GemvTensor &gt, uint32_t m, Prio &pr,
                                           int32_t *__restrict__ status) {
    const uint8_t *region = blob + ch.byte_offset;
    uint32_t x = reinterpret_cast<const uint32_t *>(region)[lane];
    Stream s;
    ring_open(s, region + kStateBytes, lds_addr(ring_lds), ch.n_words, lane);
    const uint32_t full_blocks = ch.n_symbols / kBlockSyms;  // whole rows
    const uint32_t row_blocks = cols / kBlockSyms;
    const uint8_t *sm_g = signmant + ch.out_elem;
    uint32_t smr[kSmAhead] = {};
    if (SPLIT)
#pragma unroll
        for (uint32_t j = 0; j < kSmAhead; ++j)
            if (j < full_blocks) smr[j] = load_sm4(sm_g + j * kBlockSyms, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): states, first ring units
    s.landed = s.issued;
    ring_horizon(s);

    uint64_t row = ch.scale_row - gt.row0;  // weight row of the tensor
    const float *scale_row = scales + ch.scale_row;
    float scale = SPLIT ? 0.f : *scale_row;
    const uint16_t *xa = gt.x + 4u * lane;  // this lane's columns of block 0
    uint32_t kb = 0;                        // block within the row
    float acc[M];
#pragma unroll
    for (int g = 0; g < M; ++g) acc[g] = 0.f;

    auto block = [&](uint32_t b, uint32_t &sm_reg) __attribute__((always_inline)) {
        if (PRIO) pr.tick();
        if (__builtin_expect(s.pos > s.hpos, 0)) ring_service(s, lane);
        // the block's activation columns (in flight while it decodes; at
        // least one load follows every ring refill, as ring_service's wait
        // for all but the latest operation requires)
        uint2 a[M];
#pragma unroll
        for (int g = 0; g < M; ++g)
            a[g] = ((uint32_t)g < m) ? *reinterpret_cast<const uint2 *>(
                                          xa + (uint64_t)g * gt.ldx + (uint64_t)kb * kBlockSyms)
                                    : make_uint2(0, 0);
#pragma unroll
        for (uint32_t t = 0; t < kBlockSteps; ++t)
            stream_step<false>(x, s.pos, T, stage + 64u * t, lane, true);
        // lane k: weights of columns 4k .. 4k+3 of the block, as bf16 pairs
        const uint2 d = *reinterpret_cast<const uint2 *>(stage + 4u * lane);
        uint2 w;
        if (SPLIT) {
            w = make_uint2(merge2(__builtin_amdgcn_perm(d.x, sm_reg, 0x07010500u)),
                           merge2(__builtin_amdgcn_perm(d.y, sm_reg, 0x07030502u)));
            // block b + kSmAhead's bytes into the register just consumed (past
            // the last block: this block's again, unused), kept after the merge
            __builtin_amdgcn_sched_barrier(0);
            sm_reg = load_sm4(sm_g + (b + kSmAhead < full_blocks ? kSmAhead * kBlockSyms : 0u),
                              lane);
            sm_g += kBlockSyms;
        } else {
            w = make_uint2(dequant2<E4M3>(d.x, scale), dequant2<E4M3>(d.y, scale));
        }
#pragma unroll
        for (int g = 0; g < M; ++g) acc[g] = dot2_bf16(w.y, a[g].y, dot2_bf16(w.x, a[g].x, acc[g]));
        if (__builtin_expect(++kb == row_blocks, 0)) {  // b ends a weight row
#pragma unroll
            for (int g = 0; g < M; ++g) {
                const float v = wave_sum(acc[g]);
                if (lane == 0 && (uint32_t)g < m) gt.y[(uint64_t)g * gt.ldy + row] = v;
                acc[g] = 0.f;
            }
            kb = 0;
            ++row;
            if (!SPLIT && b + 1 < full_blocks) scale = *++scale_row;
        }
    };
    uint32_t b = 0;
    if (SPLIT) {
        for (; b + kSmAhead <= full_blocks; b += kSmAhead)
#pragma unroll
            for (uint32_t j = 0; j < kSmAhead; ++j) block(b + j, smr[j]);
#pragma unroll
        for (uint32_t j = 0; j < kSmAhead; ++j)
            if (b + j < full_blocks) block(b + j, smr[j]);
    } else {
        for (; b < full_blocks; ++b) block(b, smr[0]);
    }
    const uint64_t bad_state = __ballot(x != kStateLow);
    if (status && lane == 0)
        status[ch.status_index] = (ring_consumed(s) != s.nw) ? ENTQ_CHUNK_BAD_WORDS
                                  : (bad_state ? ENTQ_CHUNK_BAD_STATE : ENTQ_CHUNK_OK);
    wait_vm<0>();  // no global->LDS load may outlive the chunk
}

// M: activation rows the kernel is built for (m <= M rows are used).
template <int M, bool SPLIT, bool PRIO>
__global__ __launch_bounds__(kThreads) ENTQ_TWO_WORKGROUPS_SGPRS void decode_gemv(
    const SlotEntry *__restrict__ tables, const DevTensor *__restrict__ tensors,
    const DevChunk *__restrict__ chunks, const DevTask *__restrict__ tasks,
    const uint8_t *__restrict__ blob, const float *__restrict__ scales,
    const uint8_t *__restrict__ signmant, int32_t *__restrict__ status, GemvArgs args) {
    __shared__ __attribute__((aligned(16))) uint16_t RING[kWaves][kRingWords];
    __shared__ uint2 T[kProbScale];
    __shared__ WaveStage STG[kWaves];

    const DevTask task = tasks[blockIdx.x];
    const bool e4m3 = tensors[task.tensor].kind == ENTQ_SYM_E4M3;
    const uint32_t cols = tensors[task.tensor].cols;
    const GemvTensor &gt = args.t[task.tensor];
    load_table(T, tables, task.tensor);
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    // the task's chunks in rounds of equal width, as in decode_stream
    const uint32_t rounds = (task.n_chunks + kWaves - 1) / kWaves;
    const uint32_t width = (task.n_chunks + rounds - 1) / rounds;
    Prio pr = {};
    if (PRIO) {
        uint32_t my_blocks = 0;
        for (uint32_t c = wave; wave < width && c < task.n_chunks; c += width)
            my_blocks += chunks[task.first_chunk + c].n_symbols / kBlockSyms;
        pr.start(my_blocks);
    }
    for (uint32_t c = wave; wave < width && c < task.n_chunks; c += width) {
        const DevChunk ch = chunks[task.first_chunk + c];
        if (SPLIT)
            gemv_chunk<M, false, true, PRIO>(ch, blob, T, RING[wave], STG[wave].stage, lane, cols,
                                             scales, signmant, gt, args.m, pr, status);
        else if (e4m3)
            gemv_chunk<M, true, false, PRIO>(ch, blob, T, RING[wave], STG[wave].stage, lane, cols,
                                             scales, signmant, gt, args.m, pr, status);
        else
            gemv_chunk<M, false, false, PRIO>(ch, blob, T, RING[wave], STG[wave].stage, lane,
                                              cols, scales, signmant, gt, args.m, pr, status);
    }
}

template <int M, bool SPLIT>
void launch_gemv_m(bool prio, dim3 grid, hipStream_t st, const entq_plan_t *plan,
                   const uint8_t *blob, const float *scales, const uint8_t *signmant,
                   int32_t *status, const GemvArgs &args) {
    const dim3 block(kThreads);
    if (prio)
        hipLaunchKernelGGL((decode_gemv<M, SPLIT, true>), grid, block, 0, st, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, blob, scales, signmant,
                           status, args);
    else
        hipLaunchKernelGGL((decode_gemv<M, SPLIT, false>), grid, block, 0, st, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, blob, scales, signmant,
                           status, args);
}

template <bool SPLIT>
void launch_gemv(int m, bool prio, dim3 grid, hipStream_t st, const entq_plan_t *plan,
                 const uint8_t *blob, const float *scales, const uint8_t *signmant,
                 int32_t *status, const GemvArgs &args) {
    static_assert(kGemvMaxRows == 4, "kernels for 1, 2 and 4 rows");
    if (m == 1)
        launch_gemv_m<1, SPLIT>(prio, grid, st, plan, blob, scales, signmant, status, args);
    else if (m == 2)
        launch_gemv_m<2, SPLIT>(prio, grid, st, plan, blob, scales, signmant, status, args);
    else
        launch_gemv_m<4, SPLIT>(prio, grid, st, plan, blob, scales, signmant, status, args);
}

}  // namespace

int launch_decode_gemv(const entq_plan_t *plan, const void *blob, const float *scales,
                       const uint8_t *signmant, const entq_gemm_io *io, int m, int32_t *status,
                       void *stream) {
    if (m < 1 || m > kGemvMaxRows || plan->n_tensors > kGemvMaxTensors ||
        plan->n_tasks > 0x7FFFFFFF)
        return ENTQ_EINVAL;
    if (plan->n_tasks == 0) return ENTQ_OK;
    GemvArgs args = {};
    args.m = (uint32_t)m;
    for (int t = 0; t < plan->n_tensors; ++t) {
        const HostTensor &h = plan->host_tensors[(size_t)t];
        if (h.n_symbols == 0) continue;
        args.t[t] = {static_cast<const uint16_t *>(io[t].d_x), io[t].d_y, io[t].ldx, io[t].ldy,
                     h.scale_row_offset};
    }
    // the priority pays off once workgroups run several chunks per wave
    const bool prio = plan->n_chunks > plan->n_tasks;
    const dim3 grid((unsigned)plan->n_tasks);
    const hipStream_t st = (hipStream_t)stream;
    const uint8_t *b = static_cast<const uint8_t *>(blob);
    if (signmant)
        launch_gemv<true>(m, prio, grid, st, plan, b, scales, signmant, status, args);
    else
        launch_gemv<false>(m, prio, grid, st, plan, b, scales, signmant, status, args);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

}  // namespace entq

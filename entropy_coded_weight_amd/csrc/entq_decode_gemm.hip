// entq_decode_gemm.hip -- gfx950 kernel that decodes compressed weight
// tensors and multiplies them with a few rows of activations in one pass,
// without writing the decoded bf16 weights anywhere.
//
// The pages expect dedicated fused kernels to make entropy-coded weights
// cheaper at inference [EntQuant, "Float8@2bits: Entropy Coding Enables
// Data-Free Model Compression", technical summary §5], and the discussion of
// the DFloat11 write-up suggests a matrix multiply that decompresses each
// tile as it goes. For each tensor W [rows x cols] of a plan this computes
//     Y [m x rows] = X [m x cols] . bf16(W)^T      (fp32 accumulation)
// where bf16(W) are exactly the values the bf16 decode would write.
//
// Mapping onto CDNA4. A chunk holds whole rows (chunk size a multiple of
// cols), so the chunks of a tensor start at row boundaries and, after the
// same number of steps, every chunk is at the same column of one of its
// rows. A workgroup of 16 waves decodes 16 consecutive chunks of one tensor
// in lockstep, 4 steps (256 columns) per block, each wave into its own LDS
// row: after a block the workgroup holds a 16-row x 256-column weight tile.
// Each wave then multiplies a 16-column slice of it (its wave index picks
// the slice) with the matching activation columns on the matrix cores,
// v_mfma_f32_16x16x16_bf16 (A = 16 activation rows, m <= 64 rows in up to
// four groups, the last padded with zeros; B = the slice, one column per
// weight row), accumulating in fp32.
// At the end of each weight row the 16 waves' partial sums are added in LDS
// (fixed order) and written out.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "entq.h"
#include "entq_internal.h"
#include "entq_stream.h"

namespace entq {
namespace {

constexpr int kGemmMaxTensors = 16;  // tensors per launch
constexpr uint32_t kGemmM = 16;      // activation rows of one MFMA tile
constexpr int kGemmMaxGroups = 4;    // up to 64 activation rows per launch

struct GemmTensor {
    const uint16_t *x;   // bf16 activations (row-major, ldx), or their packed copy
    float *y;
    uint64_t ldx, ldy;   // row strides in elements
    uint32_t chunk_base; // first DevChunk of the tensor
    uint32_t n_chunks;
    uint32_t group0;     // first workgroup of the tensor in this launch
    uint32_t table;      // the tensor's index in the plan (its slot table)
    uint32_t cols;
    uint32_t rows_per_chunk;
    uint32_t e4m3;
    uint32_t rows;       // weight rows of the tensor
};

struct GemmArgs {
    GemmTensor t[kGemmMaxTensors];
    uint32_t n_tensors;
    uint32_t m;
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// MT: groups of 16 activation rows. SPLIT: the weights are BF16 rebuilt from
// a coded exponent stream and raw sign+mantissa bytes (no scales). PACKED:
// x is the packed copy written by pack_activations (below), so each wave's
// activation fragments of a block are one contiguous run of MT x 512 bytes
// instead of 16 rows x 32 bytes per group.
template <int MT, bool SPLIT, bool PACKED>
__global__ __launch_bounds__(kThreads) ENTQ_TWO_WORKGROUPS_SGPRS void decode_gemm(const SlotEntry *__restrict__ tables,
                                                        const DevChunk *__restrict__ chunks,
                                                        const uint8_t *__restrict__ blob,
                                                        const float *__restrict__ scales,
                                                        const uint8_t *__restrict__ signmant,
                                                        int32_t *__restrict__ status,
                                                        GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint16_t RING[kWaves][kRingWords];
    __shared__ uint2 T[kProbScale];
    // two tiles of 16 weight rows x 256 columns (bf16), used in turn; at the
    // end of a weight row the same bytes hold the 16 waves' partial sums
    __shared__ __attribute__((aligned(16))) uint16_t TILE[2][kWaves][kBlockSyms];
    static_assert(sizeof(TILE) >= kWaves * 256 * sizeof(float), "partial sums fit the tiles");

    uint32_t ti = 0;
    while (ti + 1 < args.n_tensors && args.t[ti + 1].group0 <= blockIdx.x) ++ti;
    const GemmTensor &gt = args.t[ti];
    load_table(T, tables, gt.table);

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t first = (blockIdx.x - gt.group0) * kWaves;  // this group's first chunk
    const bool has_chunk = first + wave < gt.n_chunks;
    const uint32_t cols = gt.cols;
    const uint32_t blocks_per_row = cols / kBlockSyms;

    DevChunk ch = {};
    uint32_t my_rows = 0;  // weight rows in this wave's chunk
    Stream s = {};
    uint32_t x = 0;
    if (has_chunk) {
        ch = chunks[gt.chunk_base + first + wave];
        my_rows = ch.n_symbols / cols;
        const uint8_t *region = blob + ch.byte_offset;
        x = reinterpret_cast<const uint32_t *>(region)[lane];
        ring_open(s, region + kStateBytes, lds_addr(RING[wave]), ch.n_words, lane);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): states and the first ring units
    s.landed = s.issued;
    ring_horizon(s);
    __syncthreads();  // the slot table

    // A operand: activation row (lane mod 16) of each group of 16, columns
    // 4 (lane / 16) .. +3 of this wave's 16-column slice of each block
    const uint32_t a_row = lane & 15;
    const uint16_t *xa = gt.x + (uint64_t)a_row * gt.ldx + 16u * wave + 4u * (lane >> 4);
    const uint64_t group_stride = 16ull * gt.ldx;
    // B operand: weight row (lane mod 16) of the tile, same columns
    const uint32_t b_off = (lane & 15) * kBlockSyms + 16u * wave + 4u * (lane >> 4);
    const uint32_t rows_per_chunk = gt.rows_per_chunk;

    for (uint32_t r = 0; r < rows_per_chunk; ++r) {
        const bool live = r < my_rows;  // uniform per wave
        const float scale = (live && !SPLIT) ? scales[ch.scale_row + r] : 0.f;
        // sign+mantissa bytes of this lane's four columns of each block of
        // the row: block kb's are loaded into register smr[kb % kSmAhead]
        // kSmAhead blocks ahead of their use (the block loop is unrolled
        // kSmAhead times so that the registers are never copied: a copy
        // would wait for the load in flight)
        // (a wave past its rows reads the buffer's first row instead, unused:
        // every wave issues the same loads, so that the compiler's wait
        // counts stay exact)
        const uint8_t *sm_row = signmant + (live ? ch.out_elem + (uint64_t)r * cols : 0);
        uint32_t smr[kSmAhead] = {};
        if (SPLIT)
#pragma unroll
            for (uint32_t j = 0; j < kSmAhead; ++j)
                if (j < blocks_per_row) smr[j] = load_sm4(sm_row + j * kBlockSyms, lane);
        float4_t acc[MT];
#pragma unroll
        for (int g = 0; g < MT; ++g) acc[g] = float4_t{0.f, 0.f, 0.f, 0.f};
        auto block = [&](uint32_t kb, uint32_t &sm_reg) __attribute__((always_inline)) {
            const uint32_t buf = kb & 1;
            uint16_t *row_tile = TILE[buf][wave];
            if (live) {
                if (__builtin_expect(s.pos > s.hpos, 0)) ring_service(s, lane);
            }
            // this block's activation slices (in flight while the block decodes)
            uint2 a[MT];
#pragma unroll
            for (int g = 0; g < MT; ++g) {
                a[g] = make_uint2(0, 0);
                if (PACKED)  // rows past m are zeros in the packed copy
                    a[g] = *reinterpret_cast<const uint2 *>(
                        gt.x + (((uint64_t)kb * kWaves + wave) * MT + g) * 256u + 4u * lane);
                else if (SPLIT) {  // unconditional (row 0 past m, then zeroed)
                    const bool in_m = 16u * g + a_row < args.m;
                    const uint2 v = *reinterpret_cast<const uint2 *>(
                        (in_m ? xa + g * group_stride : xa - (uint64_t)a_row * gt.ldx) +
                        (uint64_t)kb * kBlockSyms);
                    a[g] = in_m ? v : make_uint2(0, 0);
                } else if (16u * g + a_row < args.m)
                    a[g] = *reinterpret_cast<const uint2 *>(xa + g * group_stride +
                                                            (uint64_t)kb * kBlockSyms);
            }
            if (live) {
                // Priority falls as a wave works through the block's steps, so that
                // the waves behind -- the ones the workgroup will wait for at the
                // block's barrier -- win issue against those ahead and against the
                // other workgroup on the CU (573.6 -> 563.7 us per 70B-shaped layer
                // at m = 16).
                static_assert(kBlockSteps == 4, "one priority level per step");
                __builtin_amdgcn_s_setprio(3);
                stream_step<false>(x, s.pos, T, row_tile, lane, true);
                __builtin_amdgcn_s_setprio(2);
                stream_step<false>(x, s.pos, T, row_tile + 64u, lane, true);
                __builtin_amdgcn_s_setprio(1);
                stream_step<false>(x, s.pos, T, row_tile + 128u, lane, true);
                __builtin_amdgcn_s_setprio(0);
                stream_step<false>(x, s.pos, T, row_tile + 192u, lane, true);
                // lane k: columns 4k .. 4k+3 of the block, made bf16 in place
                const uint2 d = *reinterpret_cast<const uint2 *>(row_tile + 4u * lane);
                uint2 w;
                if (SPLIT)  // per 16-bit half: exponent << 8 | sign+mantissa
                    w = make_uint2(merge2(__builtin_amdgcn_perm(d.x, sm_reg, 0x07010500u)),
                                   merge2(__builtin_amdgcn_perm(d.y, sm_reg, 0x07030502u)));
                else if (gt.e4m3)
                    w = make_uint2(dequant2<true>(d.x, scale), dequant2<true>(d.y, scale));
                else
                    w = make_uint2(dequant2<false>(d.x, scale), dequant2<false>(d.y, scale));
                *reinterpret_cast<uint2 *>(row_tile + 4u * lane) = w;
            } else {
                *reinterpret_cast<uint2 *>(row_tile + 4u * lane) = make_uint2(0, 0);
            }
            if (SPLIT) {
                // block kb + kSmAhead's bytes into the register just consumed
                // (past the row's end: this block's again, unused), by every
                // wave and after the merge, so that the register is reused in
                // place
                __builtin_amdgcn_sched_barrier(0);
                sm_reg = load_sm4(sm_row + (kb + kSmAhead < blocks_per_row ? kb + kSmAhead : kb) *
                                               kBlockSyms,
                                  lane);
            }
            __syncthreads();  // the tile of this block is complete
            const uint2 bw = *reinterpret_cast<const uint2 *>(&TILE[buf][0][0] + b_off);
#pragma unroll
            for (int g = 0; g < MT; ++g)
                acc[g] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                    __builtin_bit_cast(short4_t, a[g]), __builtin_bit_cast(short4_t, bw), acc[g],
                    0, 0, 0);
        };
        uint32_t kb = 0;
        if (SPLIT) {
            for (; kb + kSmAhead <= blocks_per_row; kb += kSmAhead)
#pragma unroll
                for (uint32_t j = 0; j < kSmAhead; ++j) block(kb + j, smr[j]);
#pragma unroll
            for (uint32_t j = 0; j < kSmAhead; ++j)
                if (kb + j < blocks_per_row) block(kb + j, smr[j]);
        } else {
            for (; kb < blocks_per_row; ++kb) block(kb, smr[0]);
        }
        // end of a weight row: add the 16 waves' partial sums, fixed order,
        // one group of activation rows at a time
        float *part = reinterpret_cast<float *>(&TILE[0][0][0]);
#pragma unroll
        for (int g = 0; g < MT; ++g) {
            __syncthreads();  // the tiles (or the previous group's sums) are read
            *reinterpret_cast<float4_t *>(part + 256u * wave + 4u * lane) = acc[g];
            __syncthreads();
            if (threadIdx.x < 256) {
                const uint32_t e = threadIdx.x;  // element of the 16x16 result
                float sum = 0.f;
                for (uint32_t w = 0; w < (uint32_t)kWaves; ++w) sum += part[256u * w + e];
                // lane l of a wave held rows 4 (l / 16) + i, column l mod 16
                const uint32_t l = e >> 2, i = e & 3;
                const uint32_t mrow = 16u * g + 4u * (l >> 4) + i;  // activation row
                const uint32_t c = l & 15;                          // chunk of the group
                const uint64_t wrow = (uint64_t)(first + c) * rows_per_chunk + r;  // weight row
                if (mrow < args.m && first + c < gt.n_chunks && wrow < gt.rows)
                    gt.y[(uint64_t)mrow * gt.ldy + wrow] = sum;
            }
        }
        __syncthreads();  // the partial sums are read before the next tile
    }
    if (has_chunk) {
        const uint64_t bad_state = __ballot(x != kStateLow);
        if (status && lane == 0)
            status[ch.status_index] = (ring_consumed(s) != s.nw) ? ENTQ_CHUNK_BAD_WORDS
                                      : (bad_state ? ENTQ_CHUNK_BAD_STATE : ENTQ_CHUNK_OK);
    }
    wait_vm<0>();  // no global->LDS load may outlive the workgroup
}

template <bool SPLIT, bool PACKED>
void launch_groups(int groups_m, dim3 grid, hipStream_t st, const entq_plan_t *plan,
                   const uint8_t *blob, const float *scales, const uint8_t *signmant,
                   int32_t *status, const GemmArgs &args) {
    const dim3 block(kThreads);
    if (groups_m == 1)
        hipLaunchKernelGGL((decode_gemm<1, SPLIT, PACKED>), grid, block, 0, st, plan->d_tables,
                           plan->d_chunks, blob, scales, signmant, status, args);
    else if (groups_m == 2)
        hipLaunchKernelGGL((decode_gemm<2, SPLIT, PACKED>), grid, block, 0, st, plan->d_tables,
                           plan->d_chunks, blob, scales, signmant, status, args);
    else if (groups_m == 3)
        hipLaunchKernelGGL((decode_gemm<3, SPLIT, PACKED>), grid, block, 0, st, plan->d_tables,
                           plan->d_chunks, blob, scales, signmant, status, args);
    else
        hipLaunchKernelGGL((decode_gemm<4, SPLIT, PACKED>), grid, block, 0, st, plan->d_tables,
                           plan->d_chunks, blob, scales, signmant, status, args);
}

// The packed copy of one tensor's activations: for block kb (256 columns),
// wave w, group g and lane l, the 8 bytes the wave's A operand takes, at
// element ((kb * 16 + w) * MT + g) * 256 + 4 l: row 16 g + (l mod 16),
// columns 256 kb + 16 w + 4 (l / 16) .. +3, zeros for rows m and beyond.
// One thread per 8 bytes, consecutive threads reading consecutive columns.
struct PackTensor {
    const uint16_t *x;
    uint16_t *xp;
    uint64_t ldx;
    uint32_t cols, first_block;
};
struct PackArgs {
    PackTensor t[kGemmMaxTensors];
    uint32_t n_tensors, m, groups;
};

__global__ __launch_bounds__(256) void pack_activations(PackArgs args) {
    uint32_t ti = 0;
    while (ti + 1 < args.n_tensors && args.t[ti + 1].first_block <= blockIdx.x) ++ti;
    const PackTensor &pt = args.t[ti];
    const uint64_t i = (uint64_t)(blockIdx.x - pt.first_block) * 256 + threadIdx.x;
    const uint32_t quads = pt.cols / 4;
    const uint64_t r = i / quads;               // activation row
    if (r >= 16ull * args.groups) return;
    const uint32_t c4 = (uint32_t)(i % quads);  // column quad
    uint2 v = make_uint2(0, 0);
    if (r < args.m) v = *reinterpret_cast<const uint2 *>(pt.x + r * pt.ldx + 4ull * c4);
    const uint32_t kb = c4 / 64, q = c4 % 64;
    const uint32_t w = q / 4, lane = (q % 4) * 16 + (uint32_t)(r % 16), g = (uint32_t)(r / 16);
    *reinterpret_cast<uint2 *>(pt.xp + (((uint64_t)kb * kWaves + w) * args.groups + g) * 256u +
                               4u * lane) = v;
}

}  // namespace

// Bytes of one tensor's packed activations (16-row groups, 256-byte aligned).
uint64_t packed_bytes(uint32_t cols, int groups_m) {
    return ((uint64_t)16 * groups_m * cols * 2 + 255) & ~(uint64_t)255;
}

int launch_pack_activations(const entq_plan_t *plan, const entq_gemm_io *io, int m,
                            const uint64_t *offsets, uint8_t *workspace, void *stream) {
    const int groups_m = (m + (int)kGemmM - 1) / (int)kGemmM;
    PackArgs pack = {};
    pack.m = (uint32_t)m;
    pack.groups = (uint32_t)groups_m;
    uint64_t blocks = 0;
    auto flush = [&]() -> int {
        if (pack.n_tensors)
            hipLaunchKernelGGL(pack_activations, dim3((unsigned)blocks), dim3(256), 0,
                               (hipStream_t)stream, pack);
        pack.n_tensors = 0;
        blocks = 0;
        return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
    };
    for (int t = 0; t < plan->n_tensors; ++t) {
        const HostTensor &h = plan->host_tensors[(size_t)t];
        if (h.n_symbols == 0) continue;
        const uint64_t pb = ((uint64_t)16 * groups_m * (h.cols / 4) + 255) / 256;
        if (pack.n_tensors == (uint32_t)kGemmMaxTensors || blocks + pb > 0x7FFFFFFFull) {
            const int r = flush();
            if (r != ENTQ_OK) return r;
        }
        pack.t[pack.n_tensors++] = {static_cast<const uint16_t *>(io[t].d_x),
                                    reinterpret_cast<uint16_t *>(workspace + offsets[t]),
                                    io[t].ldx, h.cols, (uint32_t)blocks};
        blocks += pb;
    }
    return flush();
}

uint64_t gemm_workspace_bytes(const entq_plan_t *plan, int m) {
    const int groups_m = (m + (int)kGemmM - 1) / (int)kGemmM;
    uint64_t total = 0;
    for (int t = 0; t < plan->n_tensors; ++t)
        if (plan->host_tensors[t].n_symbols)
            total += packed_bytes(plan->host_tensors[t].cols, groups_m);
    return total;
}

int launch_decode_gemm(const entq_plan_t *plan, const void *blob, const float *scales,
                       const uint8_t *signmant, const entq_gemm_io *io, int m,
                       uint8_t *workspace, int32_t *status, void *stream) {
    // a few activation rows: the product on the vector units, waves free of
    // one another (no tiles, no barrier), and no workspace
    if (m <= kGemvMaxRows && plan->n_tensors <= kGemvMaxTensors)
        return launch_decode_gemv(plan, blob, scales, signmant, io, m, status, stream);
    GemmArgs args = {};
    args.m = (uint32_t)m;
    PackArgs pack = {};
    pack.m = (uint32_t)m;
    uint64_t blocks = 0, pack_blocks = 0, ws_off = 0;
    const int groups_m = (m + (int)kGemmM - 1) / (int)kGemmM;
    pack.groups = (uint32_t)groups_m;
    const hipStream_t st = (hipStream_t)stream;
    auto flush = [&]() -> int {
        if (args.n_tensors == 0) return ENTQ_OK;
        const uint8_t *b = static_cast<const uint8_t *>(blob);
        const dim3 grid((unsigned)blocks);
        if (workspace) {
            hipLaunchKernelGGL(pack_activations, dim3((unsigned)pack_blocks), dim3(256), 0, st,
                               pack);
            if (signmant)
                launch_groups<true, true>(groups_m, grid, st, plan, b, scales, signmant, status,
                                          args);
            else
                launch_groups<false, true>(groups_m, grid, st, plan, b, scales, signmant, status,
                                           args);
        } else if (signmant) {
            launch_groups<true, false>(groups_m, grid, st, plan, b, scales, signmant, status, args);
        } else {
            launch_groups<false, false>(groups_m, grid, st, plan, b, scales, signmant, status,
                                        args);
        }
        args.n_tensors = 0;
        pack.n_tensors = 0;
        blocks = 0;
        pack_blocks = 0;
        return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
    };
    // Workgroups of tensors with the most symbols per chunk (the longest
    // rows) are dispatched first, so that the launch ends on short
    // workgroups: with the down projection's 3.5 times longer rows last, the
    // layer's last 512 workgroups ran alone on the GPU (581 against 575 us
    // per 70B-shaped layer at m = 16).
    std::vector<int> order((size_t)plan->n_tensors);
    for (int i = 0; i < plan->n_tensors; ++i) order[(size_t)i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
        return plan->host_tensors[(size_t)a].chunk_symbols >
               plan->host_tensors[(size_t)b].chunk_symbols;
    });
    for (const int t : order) {
        const HostTensor &h = plan->host_tensors[(size_t)t];
        if (h.n_symbols == 0) continue;
        const uint64_t groups = ((uint64_t)h.n_chunks + kWaves - 1) / kWaves;
        const uint64_t pb = ((uint64_t)16 * groups_m * (h.cols / 4) + 255) / 256;
        if (args.n_tensors == (uint32_t)kGemmMaxTensors || blocks + groups > 0x7FFFFFFFull ||
            pack_blocks + pb > 0x7FFFFFFFull) {
            const int r = flush();
            if (r != ENTQ_OK) return r;
        }
        GemmTensor &g = args.t[args.n_tensors++];
        g.x = static_cast<const uint16_t *>(io[t].d_x);
        if (workspace) {
            uint16_t *xp = reinterpret_cast<uint16_t *>(workspace + ws_off);
            pack.t[pack.n_tensors++] = {g.x, xp, io[t].ldx, h.cols, (uint32_t)pack_blocks};
            pack_blocks += pb;
            ws_off += packed_bytes(h.cols, groups_m);
            g.x = xp;
        }
        g.y = io[t].d_y;
        g.ldx = io[t].ldx;
        g.ldy = io[t].ldy;
        g.chunk_base = (uint32_t)h.chunk_base;
        g.n_chunks = (uint32_t)h.n_chunks;
        g.group0 = (uint32_t)blocks;
        g.table = (uint32_t)t;
        g.cols = h.cols;
        g.rows_per_chunk = h.chunk_symbols / h.cols;
        g.e4m3 = h.kind == ENTQ_SYM_E4M3;
        g.rows = h.rows;
        blocks += groups;
    }
    return flush();
}

}  // namespace entq

// ---------------------------------------------------------------------------
// entq_decode_gemm_static: the packed activations in a file-scope device array
// ---------------------------------------------------------------------------
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops). Each GPU holds its own copy of the array
// from the library's first use on it until the process ends. Host code never
// uses the array's name as an address: the device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and kept.

static __device__ __align__(256) uint8_t scratch[ENTQ_GEMM_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device that runs `stream`.
entq_status static_scratch(void *stream, uint8_t **out) {
    int dev = 0, cur = 0;
    if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return ENTQ_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return ENTQ_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        if (hipGetDevice(&cur) != hipSuccess) return ENTQ_EHIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return ENTQ_EHIP;
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess) return ENTQ_EHIP;
        if (e != hipSuccess || !ptr || (uintptr_t)ptr % 256) return ENTQ_EHIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = static_cast<uint8_t *>(g_scratch_ptr[dev]);
    return ENTQ_OK;
}

}  // namespace

extern "C" {

namespace {

// Checks shared by both entry points; kinds_ok tells which symbol kinds the
// call takes.
entq_status check_gemm_args(const entq_plan_t *plan, const entq_gemm_io *io, int m,
                            bool split) {
    if (!plan || plan->adaptive || !io || m < 1 || m > (int)entq::kGemmM * entq::kGemmMaxGroups)
        return ENTQ_EINVAL;
    for (int t = 0; t < plan->n_tensors; ++t) {
        const entq::HostTensor &h = plan->host_tensors[t];
        if (h.n_symbols == 0) continue;
        if (split ? h.kind != ENTQ_SYM_BF16EXP
                  : (h.kind != ENTQ_SYM_INT8 && h.kind != ENTQ_SYM_E4M3))
            return ENTQ_EINVAL;
        if (h.tiles) return ENTQ_EINVAL;  // tile order: entq_decode_gemm_tiles
        if (h.cols == 0 || h.cols % entq::kBlockSyms || h.chunk_symbols % h.cols) return ENTQ_EINVAL;
        if (h.chunk_base > 0xFFFFFFFFll || h.n_chunks > 0xFFFFFFFFll) return ENTQ_EINVAL;
        const entq_gemm_io &g = io[t];
        if (!g.d_x || !g.d_y || g.ldx < h.cols || g.ldy < h.rows) return ENTQ_EINVAL;
        if ((uintptr_t)g.d_x % 8 || g.ldx % 4 || (uintptr_t)g.d_y % 4) return ENTQ_EALIGN;
    }
    return ENTQ_OK;
}

// An optional workspace for the packed activations: null, or 256-byte
// aligned and at least entq_decode_gemm_workspace_bytes.
entq_status check_workspace(const entq_plan_t *plan, int m, void *ws, uint64_t bytes) {
    if (!ws) return ENTQ_OK;
    if ((uintptr_t)ws % 256) return ENTQ_EALIGN;
    return bytes < entq::gemm_workspace_bytes(plan, m) ? ENTQ_EWORKSPACE : ENTQ_OK;
}

}  // namespace

uint64_t entq_decode_gemm_workspace_bytes(const entq_plan_t *plan, int m) {
    if (!plan || m < 1 || m > (int)entq::kGemmM * entq::kGemmMaxGroups) return 0;
    return entq::gemm_workspace_bytes(plan, m);
}

entq_status entq_decode_gemm(const entq_plan_t *plan, const void *d_compressed,
                             const float *d_scales, const entq_gemm_io *io, int m,
                             void *d_workspace, uint64_t workspace_bytes,
                             int32_t *d_chunk_status, void *stream) {
    entq_status st = check_gemm_args(plan, io, m, false);
    if (st != ENTQ_OK) return st;
    if (plan->n_chunks && (!d_compressed || !d_scales)) return ENTQ_EINVAL;
    if ((uintptr_t)d_scales % 4) return ENTQ_EALIGN;
    st = check_workspace(plan, m, d_workspace, workspace_bytes);
    if (st != ENTQ_OK) return st;
    return (entq_status)entq::launch_decode_gemm(plan, d_compressed, d_scales, nullptr, io, m,
                                                 static_cast<uint8_t *>(d_workspace),
                                                 d_chunk_status, stream);
}

entq_status entq_decode_gemm_static(const entq_plan_t *plan, const void *d_compressed,
                                    const float *d_scales, const entq_gemm_io *io, int m,
                                    int32_t *d_chunk_status, void *stream) {
    entq_status st = check_gemm_args(plan, io, m, false);
    if (st != ENTQ_OK) return st;
    if (plan->n_chunks && (!d_compressed || !d_scales)) return ENTQ_EINVAL;
    if ((uintptr_t)d_scales % 4) return ENTQ_EALIGN;
    if (entq::gemm_workspace_bytes(plan, m) > ENTQ_GEMM_STATIC_SCRATCH_BYTES) return ENTQ_ETOOLARGE;
    uint8_t *ptr = nullptr;
    st = static_scratch(stream, &ptr);
    if (st != ENTQ_OK) return st;
    // the pack kernel writes every byte the product reads (zeros for rows
    // past m), so the previous call's contents need no clearing
    return (entq_status)entq::launch_decode_gemm(plan, d_compressed, d_scales, nullptr, io, m, ptr,
                                                 d_chunk_status, stream);
}

entq_status entq_decode_gemm_bf16_split(const entq_plan_t *plan, const void *d_exp_stream,
                                        const uint8_t *d_signmant, const entq_gemm_io *io,
                                        int m, void *d_workspace, uint64_t workspace_bytes,
                                        int32_t *d_chunk_status, void *stream) {
    entq_status st = check_gemm_args(plan, io, m, true);
    if (st != ENTQ_OK) return st;
    if (plan->n_chunks && (!d_exp_stream || !d_signmant)) return ENTQ_EINVAL;
    if ((uintptr_t)d_signmant % 16) return ENTQ_EALIGN;
    for (int t = 0; t < plan->n_tensors; ++t)
        if (plan->host_tensors[t].n_symbols && plan->host_tensors[t].out_elem_offset % 16)
            return ENTQ_EALIGN;
    st = check_workspace(plan, m, d_workspace, workspace_bytes);
    if (st != ENTQ_OK) return st;
    return (entq_status)entq::launch_decode_gemm(plan, d_exp_stream, nullptr, d_signmant, io, m,
                                                 static_cast<uint8_t *>(d_workspace),
                                                 d_chunk_status, stream);
}

}  // extern "C"

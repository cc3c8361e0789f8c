// entq_decode_tiles.hip -- gfx950 kernels of the fused decode + product on
// tile-ordered chunks: every wave decodes its own chunks and feeds the
// matrix cores straight from its registers.
//
// The discussion under the DFloat11 write-up asks for a matrix multiply
// that decompresses each tile as it goes, and EntQuant expects fused kernels
// to make entropy-coded weights cheaper at inference [EntQuant,
// "Float8@2bits: Entropy Coding Enables Data-Free Model Compression",
// technical summary §5]. The pages leave the order of the symbols inside a
// coded segment open; this file reads chunks whose symbols are in tile
// order (entq_tile_order): a chunk covers 16 weight rows (a band) and C
// columns, and its stream position 256 t + 64 s + l holds the weight at row
// l mod 16 of the band and column 16 t + 4 (l div 16) + s of the chunk.
//
// Mapping onto CDNA4. Lane l decodes stream position 64 s + l at step s of
// a 4-step block, so after the block it holds, in registers, the 4 weights
// of row l mod 16 at columns 16 t + 4 (l div 16) .. +3: exactly its part of
// the B operand of v_mfma_f32_16x16x16_bf16 for that 16 x 16 tile (B[k][n]
// = W[row n][column k]). The lane dequantises them with its row's scale,
// loads the matching activation columns (A = 16 activation rows x 16
// columns) and issues one MFMA per 16 activation rows. No LDS stage, no
// workgroup barrier, no lockstep: every wave walks its own run of chunks as
// in the bf16 decode (word ring, slot table and progress priority
// unchanged). The activations are first copied into the order the waves
// read them. At a chunk's end the wave holds Y for its 16 weight rows over
// the chunk's C columns: it writes them straight to Y when the chunk spans
// all columns, else to a partial-sum slot of the workspace, and a last
// kernel adds the column chunks' partial sums in column order.
#include <hip/hip_runtime.h>

#include "entq.h"
#include "entq_internal.h"
#include "entq_stream.h"

namespace entq {
namespace {

constexpr int kTileMaxTensors = 16;   // tensors of a plan
constexpr uint32_t kTileM = 16;       // activation rows of one MFMA
constexpr int kTileMaxGroups = 4;     // up to 64 activation rows

struct TileTensor {
    const uint16_t *x;  // the packed copy of the activations (see tile_chunk)
    float *y;           // fp32 results: m rows, row stride ldy
    float *part;        // partial sums [n_cc][m][rows], when n_cc > 1
    uint64_t ldy;
    uint64_t out0;      // the tensor's first stream element (out_elem_offset)
    uint64_t row0;      // its first scale row
    uint32_t rows, chunk_cols, n_cc;
};
struct TileArgs {
    TileTensor t[kTileMaxTensors];
    uint32_t m;
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// One decode step without staging: the lane's slot-table entry (f | sym <<
// 24) is returned, the state updated and renormalised as in stream_step.
__device__ __forceinline__ uint32_t tile_step(uint32_t &x, uint32_t &pos, const uint2 *T,
                                              uint32_t lane) {
    const uint2 e = T[x & (kProbScale - 1)];
    x = __umul24(e.x, x >> kProbBits) + e.y;
    const bool need = x < kStateLow;
    const uint64_t mask = __ballot(need);
    const uint32_t w = *reinterpret_cast<lds_u16 *>((pos + lane_prefix(mask)) << 1);
    x = __builtin_amdgcn_perm(x, w, need ? 0x05040100u : 0x07060504u);
    pos += (uint32_t)__popcll(mask);
    return e.x;
}

// bf16 of two codes (bytes 1 and 3 of d) times a per-lane scale; otherwise
// as dequant2 (the code is the product's first operand, NaN codes patched).
template <bool E4M3>
__device__ __forceinline__ uint32_t dequant2_lane(uint32_t d, float scale) {
    float v0, v1;
    if (E4M3) {
        v0 = __builtin_amdgcn_cvt_f32_fp8((int)d, 1);
        v1 = __builtin_amdgcn_cvt_f32_fp8((int)d, 3);
    } else {
        v0 = (float)((int32_t)(d << 16) >> 24);
        v1 = (float)((int32_t)d >> 24);
    }
    const uint32_t r = bf16x2_bits(mul_value_scale(v0, scale), mul_value_scale(v1, scale));
    return E4M3 ? e4m3_nan_patch2(d, r) : r;
}

// The activations are read from their packed copy (launch_pack_activations):
// the A fragments of one 16-column slice and group of 16 rows are 512
// contiguous bytes, where the activations' own layout gives 16 rows of 32
// bytes (partial cache lines). Measured on 70B-shaped layers with
// 8,192-column chunks, reading X in its own layout: m = 1, 2, 4: 356.0,
// 358.5, 363.7 us, m = 16 419.8 us, m = 64 1,549 us; from the packed copy:
// m = 2 .. 16 336-343 us, m = 64 539 us (the copy included).
// SPLIT: BF16 weights from a coded exponent stream and raw sign+mantissa
// bytes, both in tile order (no scales).
template <int MT, bool E4M3, bool SPLIT, bool PRIO>
__device__ __forceinline__ void tile_chunk(const DevChunk &ch, const uint8_t *__restrict__ blob,
                                           const uint2 *T, uint16_t *ring_lds, uint32_t lane,
                                           const float *__restrict__ scales,
                                           const uint8_t *__restrict__ signmant,
                                           const TileTensor &gt, uint32_t m, Prio &pr,
                                           int32_t *__restrict__ status) {
    const uint8_t *region = blob + ch.byte_offset;
    uint32_t x = reinterpret_cast<const uint32_t *>(region)[lane];
    Stream s;
    ring_open(s, region + kStateBytes, lds_addr(ring_lds), ch.n_words, lane);
    // which band and column chunk: chunks are whole 16 x C pieces in order
    const uint32_t C = gt.chunk_cols;
    const uint64_t k = (ch.out_elem - gt.out0) / (16ull * C);
    const uint32_t band = (uint32_t)(k / gt.n_cc), cc = (uint32_t)(k % gt.n_cc);
    const uint32_t r16 = lane & 15;                  // weight row in the band; activation row
    const float scale = SPLIT ? 0.f : scales[gt.row0 + 16ull * band + r16];
    // split: this lane's sign+mantissa bytes, stream positions 64 s + l of each tile
    const uint8_t *smc = SPLIT ? signmant + ch.out_elem + lane : nullptr;
    // activations: a uniform base and 32-bit byte offsets (a packed copy
    // holds 32 x groups x cols bytes), so the loads need no 64-bit address
    // registers per group
    const uint8_t *xb = reinterpret_cast<const uint8_t *>(gt.x);
    const uint32_t xoff = 2u * ((cc * C / 16u) * MT * 256u + 4u * lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): states, scale, first ring units
    s.landed = s.issued;
    ring_horizon(s);

    float4_t acc[MT];
#pragma unroll
    for (int g = 0; g < MT; ++g) acc[g] = float4_t{0.f, 0.f, 0.f, 0.f};
    const uint32_t blocks = ch.n_symbols / kBlockSyms;  // C / 16 tiles
    for (uint32_t t = 0; t < blocks; ++t) {
        if (PRIO) pr.tick();
        if (__builtin_expect(s.pos > s.hpos, 0)) ring_service(s, lane);
        // this tile's activation columns (in flight while it decodes; at
        // least one load follows every ring refill, as ring_service's wait
        // for all but the latest operation requires)
        uint2 a[MT];
#pragma unroll
        for (int g = 0; g < MT; ++g)  // (rows m and beyond are zeros in the copy)
            a[g] = *reinterpret_cast<const uint2 *>(xb + (xoff + (t * MT + g) * 512u));
        uint32_t sm0 = 0, sm1 = 0, sm2 = 0, sm3 = 0;
        if (SPLIT) {
            const uint8_t *sp = smc + 256ull * t;
            sm0 = sp[0];
            sm1 = sp[64];
            sm2 = sp[128];
            sm3 = sp[192];
        }
        const uint32_t e0 = tile_step(x, s.pos, T, lane);
        const uint32_t e1 = tile_step(x, s.pos, T, lane);
        const uint32_t e2 = tile_step(x, s.pos, T, lane);
        const uint32_t e3 = tile_step(x, s.pos, T, lane);
        // codes of columns +0, +1 in bytes 1 and 3, then of +2, +3
        const uint32_t d0 = __builtin_amdgcn_perm(e1, e0, 0x070C030Cu);
        const uint32_t d1 = __builtin_amdgcn_perm(e3, e2, 0x070C030Cu);
        uint2 w;
        if (SPLIT)  // per 16-bit half: exponent << 8 | sign+mantissa, then bf16
            w = make_uint2(merge2((d0 & 0xFF00FF00u) | sm0 | (sm1 << 16)),
                           merge2((d1 & 0xFF00FF00u) | sm2 | (sm3 << 16)));
        else
            w = make_uint2(dequant2_lane<E4M3>(d0, scale), dequant2_lane<E4M3>(d1, scale));
#pragma unroll
        for (int g = 0; g < MT; ++g)
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                __builtin_bit_cast(short4_t, a[g]), __builtin_bit_cast(short4_t, w), acc[g], 0, 0,
                0);
    }
    // lane l holds Y[16 g + 4 (l div 16) + i][band row l mod 16], i = 0..3
    const uint32_t wrow = 16u * band + r16;
    float *dst;
    uint64_t ld;
    if (gt.n_cc > 1) {
        dst = gt.part + (uint64_t)cc * m * gt.rows;
        ld = gt.rows;
    } else {
        dst = gt.y;
        ld = gt.ldy;
    }
#pragma unroll
    for (int g = 0; g < MT; ++g)
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i) {
            const uint32_t mrow = 16u * g + 4u * (lane >> 4) + i;
            if (mrow < m) dst[(uint64_t)mrow * ld + wrow] = acc[g][i];
        }
    const uint64_t bad_state = __ballot(x != kStateLow);
    if (status && lane == 0)
        status[ch.status_index] = (ring_consumed(s) != s.nw) ? ENTQ_CHUNK_BAD_WORDS
                                  : (bad_state ? ENTQ_CHUNK_BAD_STATE : ENTQ_CHUNK_OK);
    wait_vm<0>();  // no global->LDS load may outlive the chunk
}

// amdgpu_waves_per_eu(8): at most 64 vector registers per lane, so that two
// 16-wave workgroups share a CU also with four 16-row groups of activations
// (the compiler would otherwise take 78 there and halve the waves).
template <int MT, bool PRIO, bool SPLIT>
__global__ __launch_bounds__(kThreads) ENTQ_TWO_WORKGROUPS_SGPRS
__attribute__((amdgpu_waves_per_eu(8, 8))) void decode_tile_gemm(
    const SlotEntry *__restrict__ tables, const DevTensor *__restrict__ tensors,
    const DevChunk *__restrict__ chunks, const DevTask *__restrict__ tasks,
    const uint8_t *__restrict__ blob, const float *__restrict__ scales,
    const uint8_t *__restrict__ signmant, int32_t *__restrict__ status, TileArgs args) {
    __shared__ __attribute__((aligned(16))) uint16_t RING[kWaves][kRingWords];
    __shared__ uint2 T[kProbScale];

    const DevTask task = tasks[blockIdx.x];
    const bool e4m3 = tensors[task.tensor].kind == ENTQ_SYM_E4M3;
    const TileTensor &gt = args.t[task.tensor];
    load_table(T, tables, task.tensor);
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    // the task's chunks in rounds of equal width, as in the bf16 decode
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
            tile_chunk<MT, false, true, PRIO>(ch, blob, T, RING[wave], lane, scales, signmant, gt,
                                              args.m, pr, status);
        else if (e4m3)
            tile_chunk<MT, true, false, PRIO>(ch, blob, T, RING[wave], lane, scales, signmant, gt,
                                              args.m, pr, status);
        else
            tile_chunk<MT, false, false, PRIO>(ch, blob, T, RING[wave], lane, scales, signmant,
                                               gt, args.m, pr, status);
    }
}

// ---------------------------------------------------------------------------
// decode of tile-ordered tensors into their row-major outputs
// ---------------------------------------------------------------------------
//
// The same walk over a chunk's tiles, so that a tensor kept in tile order
// for the fused product also decodes to the ordinary row-major weights.
// After a tile each lane holds 4 consecutive outputs of one row; two tiles
// are staged per wave in LDS (16 rows x 32 columns) and leave as 16 rows of
// 64 contiguous bytes (bf16; 32 for codes), one 16-byte (8-byte) store per
// lane. (Storing each tile straight from the lanes, 16 rows of 32 bytes:
// 971 us per 70B-shaped layer against 456 us for the row-major decode.)
template <int MODE, bool E4M3, bool PRIO>
__device__ __forceinline__ void tile_decode_chunk(const DevChunk &ch,
                                                  const uint8_t *__restrict__ blob,
                                                  const uint2 *T, uint16_t *ring_lds,
                                                  uint16_t *stage, uint32_t lane,
                                                  const float *__restrict__ scales,
                                                  const uint8_t *__restrict__ signmant,
                                                  const TileTensor &gt, void *__restrict__ out,
                                                  Prio &pr, int32_t *__restrict__ status) {
    const uint8_t *region = blob + ch.byte_offset;
    uint32_t x = reinterpret_cast<const uint32_t *>(region)[lane];
    Stream s;
    ring_open(s, region + kStateBytes, lds_addr(ring_lds), ch.n_words, lane);
    const uint32_t C = gt.chunk_cols;
    const uint64_t k = (ch.out_elem - gt.out0) / (16ull * C);
    const uint32_t band = (uint32_t)(k / gt.n_cc), cc = (uint32_t)(k % gt.n_cc);
    const uint32_t r16 = lane & 15;
    const uint64_t cols = (uint64_t)gt.n_cc * C;
    const float scale = (MODE == kModeBf16) ? scales[gt.row0 + 16ull * band + r16] : 0.f;
    const uint8_t *smc = (MODE == kModeSplit) ? signmant + ch.out_elem + lane : nullptr;
    // this lane's first output: row 16 band + r16, column cC + 4 (lane / 16);
    // and its staged run of a pair of tiles: row lane / 4, columns 8 (lane % 4) ..
    const uint64_t o0 = gt.out0 + (16ull * band + r16) * cols + (uint64_t)cc * C + 4u * (lane >> 4);
    const uint64_t p0 =
        gt.out0 + (16ull * band + (lane >> 2)) * cols + (uint64_t)cc * C + 8u * (lane & 3);
    // stage (16 rows x 32 columns): this lane's slot of tile j of a pair, and its run
    const uint32_t put = r16 * 32u + 4u * (lane >> 4), get = (lane >> 2) * 32u + 8u * (lane & 3);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): states, scale, first ring units
    s.landed = s.issued;
    ring_horizon(s);
    const uint32_t blocks = ch.n_symbols / kBlockSyms;
    for (uint32_t t = 0; t < blocks; ++t) {
        if (PRIO) pr.tick();
        if (__builtin_expect(s.pos > s.hpos, 0)) ring_service(s, lane);
        uint32_t sm0 = 0, sm1 = 0, sm2 = 0, sm3 = 0;
        if (MODE == kModeSplit) {
            const uint8_t *sp = smc + 256ull * t;
            sm0 = sp[0];
            sm1 = sp[64];
            sm2 = sp[128];
            sm3 = sp[192];
        }
        const uint32_t e0 = tile_step(x, s.pos, T, lane);
        const uint32_t e1 = tile_step(x, s.pos, T, lane);
        const uint32_t e2 = tile_step(x, s.pos, T, lane);
        const uint32_t e3 = tile_step(x, s.pos, T, lane);
        const uint32_t j = t & 1;                     // place in the pair
        const bool last_single = (t + 1 == blocks) && j == 0;
        if (MODE == kModeCodes) {
            // the four symbols (byte 3 of each entry) in column order
            const uint32_t v = __builtin_amdgcn_perm(e1, e0, 0x0C0C0703u) |
                               __builtin_amdgcn_perm(e3, e2, 0x07030C0Cu);
            uint8_t *st8 = reinterpret_cast<uint8_t *>(stage);
            if (last_single) {
                *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(out) + o0 + 16ull * t) = v;
            } else {
                *reinterpret_cast<uint32_t *>(st8 + put + 16u * j) = v;
                if (j == 1)
                    *reinterpret_cast<uint2 *>(static_cast<uint8_t *>(out) + p0 + 16ull * (t - 1)) =
                        *reinterpret_cast<const uint2 *>(st8 + get);
            }
        } else {
            const uint32_t d0 = __builtin_amdgcn_perm(e1, e0, 0x070C030Cu);
            const uint32_t d1 = __builtin_amdgcn_perm(e3, e2, 0x070C030Cu);
            uint2 w;
            if (MODE == kModeSplit)
                w = make_uint2(merge2((d0 & 0xFF00FF00u) | sm0 | (sm1 << 16)),
                               merge2((d1 & 0xFF00FF00u) | sm2 | (sm3 << 16)));
            else
                w = make_uint2(dequant2_lane<E4M3>(d0, scale), dequant2_lane<E4M3>(d1, scale));
            if (last_single) {
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + o0 + 16ull * t) = w;
            } else {
                *reinterpret_cast<uint2 *>(stage + put + 16u * j) = w;
                if (j == 1)
                    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + p0 + 16ull * (t - 1)) =
                        *reinterpret_cast<const uint4 *>(stage + get);
            }
        }
    }
    const uint64_t bad_state = __ballot(x != kStateLow);
    if (status && lane == 0)
        status[ch.status_index] = (ring_consumed(s) != s.nw) ? ENTQ_CHUNK_BAD_WORDS
                                  : (bad_state ? ENTQ_CHUNK_BAD_STATE : ENTQ_CHUNK_OK);
    wait_vm<0>();  // no global->LDS load may outlive the chunk
}

template <int MODE, bool PRIO>
__global__ __launch_bounds__(kThreads) ENTQ_TWO_WORKGROUPS_SGPRS void decode_tiles_rowmajor(
    const SlotEntry *__restrict__ tables, const DevTensor *__restrict__ tensors,
    const DevChunk *__restrict__ chunks, const DevTask *__restrict__ tasks,
    const uint8_t *__restrict__ blob, void *__restrict__ out, const float *__restrict__ scales,
    const uint8_t *__restrict__ signmant, int32_t *__restrict__ status, TileArgs args) {
    __shared__ __attribute__((aligned(16))) uint16_t RING[kWaves][kRingWords];
    __shared__ uint2 T[kProbScale];
    __shared__ __attribute__((aligned(16))) uint16_t STG[kWaves][16 * 32];  // two tiles

    const DevTask task = tasks[blockIdx.x];
    const bool e4m3 = tensors[task.tensor].kind == ENTQ_SYM_E4M3;
    const TileTensor &gt = args.t[task.tensor];
    load_table(T, tables, task.tensor);
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
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
        if (MODE == kModeBf16 && e4m3)
            tile_decode_chunk<MODE, true, PRIO>(ch, blob, T, RING[wave], STG[wave], lane, scales,
                                                signmant, gt, out, pr, status);
        else
            tile_decode_chunk<MODE, false, PRIO>(ch, blob, T, RING[wave], STG[wave], lane, scales,
                                                 signmant, gt, out, pr, status);
    }
}

template <int MODE>
void launch_tiles_rowmajor(bool prio, dim3 grid, hipStream_t st, const entq_plan_t *plan,
                           const uint8_t *blob, void *out, const float *scales,
                           const uint8_t *signmant, int32_t *status, const TileArgs &args) {
    const dim3 block(kThreads);
    if (prio)
        hipLaunchKernelGGL((decode_tiles_rowmajor<MODE, true>), grid, block, 0, st,
                           plan->d_tables, plan->d_tensors, plan->d_chunks, plan->d_tasks, blob,
                           out, scales, signmant, status, args);
    else
        hipLaunchKernelGGL((decode_tiles_rowmajor<MODE, false>), grid, block, 0, st,
                           plan->d_tables, plan->d_tensors, plan->d_chunks, plan->d_tasks, blob,
                           out, scales, signmant, status, args);
}

// The tile order on the device: one thread per 4 bytes of the output (a
// lane's 4 consecutive columns of one row, stream positions 64 s + l of a
// tile, s = 0..3), reading the row-major source (4 contiguous bytes) and
// writing the 4 bytes to their 4 stream positions.
__global__ __launch_bounds__(256) void tile_order_bytes(const uint8_t *__restrict__ in,
                                                        uint8_t *__restrict__ out,
                                                        uint32_t cols, uint32_t chunk_cols,
                                                        uint64_t n_quads) {
    const uint64_t q = (uint64_t)blockIdx.x * 256 + threadIdx.x;  // quad = tile, lane
    if (q >= n_quads) return;
    const uint64_t tile = q >> 6;        // tiles in stream order
    const uint32_t l = (uint32_t)(q & 63);
    const uint32_t tiles_per_chunk = chunk_cols / 16;
    const uint64_t k = tile / tiles_per_chunk;  // chunk
    const uint32_t t = (uint32_t)(tile % tiles_per_chunk);
    const uint32_t n_cc = cols / chunk_cols;
    const uint64_t band = k / n_cc, cc = k % n_cc;
    const uint64_t row = 16 * band + (l & 15);
    const uint64_t col = cc * chunk_cols + 16u * t + 4u * (l >> 4);
    const uint32_t v = *reinterpret_cast<const uint32_t *>(in + row * cols + col);
    uint8_t *dst = out + tile * 256 + l;
    dst[0] = (uint8_t)v;
    dst[64] = (uint8_t)(v >> 8);
    dst[128] = (uint8_t)(v >> 16);
    dst[192] = (uint8_t)(v >> 24);
}

// Y of the tensors whose chunks split the columns: the column chunks'
// partial sums added in column order, one thread per result.
struct ReduceTensor {
    const float *part;
    float *y;
    uint64_t ldy;
    uint32_t rows, n_cc, first_block;
};
struct ReduceArgs {
    ReduceTensor t[kTileMaxTensors];
    uint32_t n_tensors, m;
};

__global__ __launch_bounds__(256) void reduce_partials(ReduceArgs args) {
    uint32_t ti = 0;
    while (ti + 1 < args.n_tensors && args.t[ti + 1].first_block <= blockIdx.x) ++ti;
    const ReduceTensor &rt = args.t[ti];
    const uint64_t i = (uint64_t)(blockIdx.x - rt.first_block) * 256 + threadIdx.x;
    const uint64_t per_cc = (uint64_t)args.m * rt.rows;
    if (i >= per_cc) return;
    float sum = 0.f;
    for (uint32_t c = 0; c < rt.n_cc; ++c) sum += rt.part[c * per_cc + i];
    const uint64_t mrow = i / rt.rows, r = i % rt.rows;
    rt.y[mrow * rt.ldy + r] = sum;
}

template <int MT, bool SPLIT>
void launch_tiles_mt(bool prio, dim3 grid, hipStream_t st, const entq_plan_t *plan,
                     const uint8_t *blob, const float *scales, const uint8_t *signmant,
                     int32_t *status, const TileArgs &args) {
    const dim3 block(kThreads);
    if (prio)
        hipLaunchKernelGGL((decode_tile_gemm<MT, true, SPLIT>), grid, block, 0, st,
                           plan->d_tables, plan->d_tensors, plan->d_chunks, plan->d_tasks, blob,
                           scales, signmant, status, args);
    else
        hipLaunchKernelGGL((decode_tile_gemm<MT, false, SPLIT>), grid, block, 0, st,
                           plan->d_tables, plan->d_tensors, plan->d_chunks, plan->d_tasks, blob,
                           scales, signmant, status, args);
}

template <bool SPLIT>
void launch_tiles(int groups, bool prio, dim3 grid, hipStream_t st, const entq_plan_t *plan,
                  const uint8_t *blob, const float *scales, const uint8_t *signmant,
                  int32_t *status, const TileArgs &args) {
    if (groups == 1)
        launch_tiles_mt<1, SPLIT>(prio, grid, st, plan, blob, scales, signmant, status, args);
    else if (groups == 2)
        launch_tiles_mt<2, SPLIT>(prio, grid, st, plan, blob, scales, signmant, status, args);
    else if (groups == 3)
        launch_tiles_mt<3, SPLIT>(prio, grid, st, plan, blob, scales, signmant, status, args);
    else
        launch_tiles_mt<4, SPLIT>(prio, grid, st, plan, blob, scales, signmant, status, args);
}

uint64_t part_bytes(const HostTensor &h, int m) {
    const uint32_t C = h.chunk_symbols / 16;
    const uint32_t ncc = h.cols / C;
    if (ncc <= 1) return 0;
    return ((uint64_t)ncc * m * h.rows * 4 + 255) & ~(uint64_t)255;
}

// Workspace: the packed activations, then the partial sums, tensor by tensor
// in plan order.
uint64_t tiles_workspace_bytes(const entq_plan_t *plan, int m) {
    const int groups = (m + (int)kTileM - 1) / (int)kTileM;
    uint64_t total = 0;
    for (int t = 0; t < plan->n_tensors; ++t) {
        const HostTensor &h = plan->host_tensors[(size_t)t];
        if (h.n_symbols == 0) continue;
        total += packed_bytes(h.cols, groups) + part_bytes(h, m);
    }
    return total;
}

entq_status check_tiles_args(const entq_plan_t *plan, const entq_gemm_io *io, int m,
                             bool split) {
    if (!plan || plan->adaptive || !io || m < 1 || m > (int)kTileM * kTileMaxGroups ||
        plan->n_tensors > kTileMaxTensors || plan->n_tasks > 0x7FFFFFFF)
        return ENTQ_EINVAL;
    for (int t = 0; t < plan->n_tensors; ++t) {
        const HostTensor &h = plan->host_tensors[(size_t)t];
        if (h.n_symbols == 0) continue;
        if (split ? h.kind != ENTQ_SYM_BF16EXP
                  : (h.kind != ENTQ_SYM_INT8 && h.kind != ENTQ_SYM_E4M3))
            return ENTQ_EINVAL;
        if (!h.tiles) return ENTQ_EINVAL;  // row-major symbols: entq_decode_gemm
        // chunks of 16 whole rows x C columns, C a multiple of 16 dividing cols
        if (h.rows % 16 || h.chunk_symbols % kBlockSyms) return ENTQ_EINVAL;
        const uint32_t C = h.chunk_symbols / 16;
        if (h.cols == 0 || h.cols % C) return ENTQ_EINVAL;
        const entq_gemm_io &g = io[t];
        if (!g.d_x || !g.d_y || g.ldx < h.cols || g.ldy < h.rows) return ENTQ_EINVAL;
        if ((uintptr_t)g.d_x % 8 || g.ldx % 4 || (uintptr_t)g.d_y % 4) return ENTQ_EALIGN;
    }
    return ENTQ_OK;
}

// Both entry points: checks done, the pack, product and reduction enqueued.
entq_status run_tiles(const entq_plan_t *plan, const void *d_compressed, const float *d_scales,
                      const uint8_t *d_signmant, const entq_gemm_io *io, int m,
                      void *d_workspace, uint64_t workspace_bytes, int32_t *d_chunk_status,
                      void *stream) {
    const uint64_t need = tiles_workspace_bytes(plan, m);
    if (need && !d_workspace) return ENTQ_EWORKSPACE;
    if (d_workspace && (uintptr_t)d_workspace % 256) return ENTQ_EALIGN;
    if (workspace_bytes < need) return ENTQ_EWORKSPACE;
    if (plan->n_tasks == 0) return ENTQ_OK;

    TileArgs args = {};
    args.m = (uint32_t)m;
    ReduceArgs red = {};
    red.m = (uint32_t)m;
    uint64_t off = 0, red_blocks = 0;
    uint8_t *ws = static_cast<uint8_t *>(d_workspace);
    const int groups = (m + (int)kTileM - 1) / (int)kTileM;
    uint64_t pack_off[kTileMaxTensors] = {};
    for (int t = 0; t < plan->n_tensors; ++t)
        if (plan->host_tensors[(size_t)t].n_symbols) {
            pack_off[t] = off;
            off += packed_bytes(plan->host_tensors[(size_t)t].cols, groups);
        }
    for (int t = 0; t < plan->n_tensors; ++t) {
        const HostTensor &h = plan->host_tensors[(size_t)t];
        if (h.n_symbols == 0) continue;
        TileTensor &g = args.t[t];
        g.x = reinterpret_cast<const uint16_t *>(ws + pack_off[t]);
        g.y = io[t].d_y;
        g.ldy = io[t].ldy;
        g.out0 = h.out_elem_offset;
        g.row0 = h.scale_row_offset;
        g.rows = h.rows;
        g.chunk_cols = h.chunk_symbols / 16;
        g.n_cc = h.cols / g.chunk_cols;
        g.part = nullptr;
        if (g.n_cc > 1) {
            g.part = reinterpret_cast<float *>(ws + off);
            off += part_bytes(h, m);
            ReduceTensor &r = red.t[red.n_tensors++];
            r = {g.part, g.y, g.ldy, g.rows, g.n_cc, (uint32_t)red_blocks};
            red_blocks += ((uint64_t)m * h.rows + 255) / 256;
        }
    }
    if (red_blocks > 0x7FFFFFFF) return ENTQ_EINVAL;
    const hipStream_t s = (hipStream_t)stream;
    const bool prio = plan->n_chunks > plan->n_tasks;
    const dim3 grid((unsigned)plan->n_tasks);
    const uint8_t *b = static_cast<const uint8_t *>(d_compressed);
    const int r = launch_pack_activations(plan, io, m, pack_off, ws, stream);
    if (r != ENTQ_OK) return (entq_status)r;
    if (d_signmant)
        launch_tiles<true>(groups, prio, grid, s, plan, b, d_scales, d_signmant, d_chunk_status,
                           args);
    else
        launch_tiles<false>(groups, prio, grid, s, plan, b, d_scales, d_signmant,
                            d_chunk_status, args);
    if (red.n_tensors)
        hipLaunchKernelGGL(reduce_partials, dim3((unsigned)red_blocks), dim3(256), 0, s, red);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

}  // namespace
}  // namespace entq

namespace entq {

int launch_tile_decode(const entq_plan_t *plan, int mode, const void *blob, void *out,
                       const float *scales, const uint8_t *signmant, int32_t *status,
                       void *stream) {
    if (plan->n_tensors > kTileMaxTensors || plan->n_tasks > 0x7FFFFFFF) return ENTQ_EINVAL;
    if (plan->n_tasks == 0) return ENTQ_OK;
    TileArgs args = {};
    for (int t = 0; t < plan->n_tensors; ++t) {
        const HostTensor &h = plan->host_tensors[(size_t)t];
        if (h.n_symbols == 0) continue;
        TileTensor &g = args.t[t];
        g.out0 = h.out_elem_offset;
        g.row0 = h.scale_row_offset;
        g.rows = h.rows;
        g.chunk_cols = h.chunk_symbols / 16;
        g.n_cc = h.cols / g.chunk_cols;
    }
    const bool prio = plan->n_chunks > plan->n_tasks;
    const dim3 grid((unsigned)plan->n_tasks);
    const hipStream_t st = (hipStream_t)stream;
    const uint8_t *b = static_cast<const uint8_t *>(blob);
    if (mode == kModeCodes)
        launch_tiles_rowmajor<kModeCodes>(prio, grid, st, plan, b, out, scales, signmant, status,
                                          args);
    else if (mode == kModeBf16)
        launch_tiles_rowmajor<kModeBf16>(prio, grid, st, plan, b, out, scales, signmant, status,
                                         args);
    else
        launch_tiles_rowmajor<kModeSplit>(prio, grid, st, plan, b, out, scales, signmant, status,
                                          args);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

}  // namespace entq

extern "C" {

uint64_t entq_decode_gemm_tiles_workspace_bytes(const entq_plan_t *plan, int m) {
    if (!plan || m < 1 || m > (int)entq::kTileM * entq::kTileMaxGroups) return 0;
    return entq::tiles_workspace_bytes(plan, m);
}

entq_status entq_decode_gemm_tiles(const entq_plan_t *plan, const void *d_compressed,
                                   const float *d_scales, const entq_gemm_io *io, int m,
                                   void *d_workspace, uint64_t workspace_bytes,
                                   int32_t *d_chunk_status, void *stream) {
    entq_status st = entq::check_tiles_args(plan, io, m, false);
    if (st != ENTQ_OK) return st;
    if (plan->n_chunks && (!d_compressed || !d_scales)) return ENTQ_EINVAL;
    if ((uintptr_t)d_scales % 4) return ENTQ_EALIGN;
    return entq::run_tiles(plan, d_compressed, d_scales, nullptr, io, m, d_workspace,
                           workspace_bytes, d_chunk_status, stream);
}

entq_status entq_decode_gemm_tiles_bf16_split(const entq_plan_t *plan, const void *d_exp_stream,
                                              const uint8_t *d_signmant, const entq_gemm_io *io,
                                              int m, void *d_workspace,
                                              uint64_t workspace_bytes, int32_t *d_chunk_status,
                                              void *stream) {
    entq_status st = entq::check_tiles_args(plan, io, m, true);
    if (st != ENTQ_OK) return st;
    if (plan->n_chunks && (!d_exp_stream || !d_signmant)) return ENTQ_EINVAL;
    return entq::run_tiles(plan, d_exp_stream, nullptr, d_signmant, io, m, d_workspace,
                           workspace_bytes, d_chunk_status, stream);
}

entq_status entq_tile_order_device(const uint8_t *d_codes, uint32_t rows, uint32_t cols,
                                   uint32_t chunk_cols, uint8_t *d_out, void *stream) {
    if (rows % 16 || chunk_cols == 0 || chunk_cols % 16 || cols % chunk_cols) return ENTQ_EINVAL;
    const uint64_t n = (uint64_t)rows * cols;
    if (n == 0) return ENTQ_OK;
    if (!d_codes || !d_out) return ENTQ_EINVAL;
    if ((uintptr_t)d_codes % 4) return ENTQ_EALIGN;
    const uint64_t quads = n / 4, blocks = (quads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return ENTQ_EINVAL;
    hipLaunchKernelGGL(entq::tile_order_bytes, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, d_codes, d_out, cols, chunk_cols, quads);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

}  // extern "C"

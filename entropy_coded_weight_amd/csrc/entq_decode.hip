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
// number of lower lanes that also read (ballot + mbcnt), the wave's pointer
// advances by the popcount. The slot table of the tensor (4096 x 8 bytes)
// sits in LDS, shared by the kWaves waves of a workgroup, which all decode
// chunks of that one tensor.
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

template <int MODE>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const SlotEntry *__restrict__ tables, const DevTensor *__restrict__ tensors,
    const DevChunk *__restrict__ chunks, const DevTask *__restrict__ tasks,
    const uint8_t *__restrict__ blob, void *__restrict__ out, const float *__restrict__ scales,
    const uint8_t *__restrict__ signmant, int32_t *__restrict__ status) {
    __shared__ uint2 T[kProbScale];
    __shared__ float V[256];

    const DevTask task = tasks[blockIdx.x];
    const DevTensor td = tensors[task.tensor];
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(tables + (size_t)task.tensor * kProbScale);
        uint4 *dst = reinterpret_cast<uint4 *>(T);
        for (uint32_t i = threadIdx.x; i < kProbScale / 2; i += kThreads) dst[i] = src[i];
        if (MODE == kModeBf16 && threadIdx.x < 256) {
            const uint32_t c = threadIdx.x;
            V[c] = (td.kind == ENTQ_SYM_E4M3) ? __builtin_amdgcn_cvt_f32_fp8((int)c, 0)
                                              : (float)(int8_t)c;
        }
    }
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
                static_cast<uint16_t *>(out)[o] = bf16_bits(V[sym] * scales[row]);
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

}  // namespace

int launch_decode(const entq_plan_t *plan, int mode, const void *blob, void *out,
                  const float *scales, const uint8_t *signmant, int32_t *status, void *stream) {
    if (plan->n_tasks == 0) return ENTQ_OK;
    if (plan->n_tasks > 0x7FFFFFFF) return ENTQ_EINVAL;
    const dim3 grid((unsigned)plan->n_tasks), block(kThreads);
    hipStream_t s = (hipStream_t)stream;
    const uint8_t *b = static_cast<const uint8_t *>(blob);
    switch (mode) {
    case kModeCodes:
        hipLaunchKernelGGL(decode_kernel<kModeCodes>, grid, block, 0, s, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, b, out, scales,
                           signmant, status);
        break;
    case kModeBf16:
        hipLaunchKernelGGL(decode_kernel<kModeBf16>, grid, block, 0, s, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, b, out, scales,
                           signmant, status);
        break;
    default:
        hipLaunchKernelGGL(decode_kernel<kModeSplit>, grid, block, 0, s, plan->d_tables,
                           plan->d_tensors, plan->d_chunks, plan->d_tasks, b, out, scales,
                           signmant, status);
        break;
    }
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

}  // namespace entq

// entq_encode_dev.hip -- gfx950 kernels of the on-device encoder: byte
// counts, the chunk-parallel 64-lane interleaved rANS encoder and the
// packer that lays the encoded chunks out as the container's regions.
//
// The method compresses each weight tensor's flattened 8-bit codes with an
// ANS coder, and the pages describe doing so with a GPU ANS library
// [EntQuant, "Float8@2bits: Entropy Coding Enables Data-Free Model
// Compression", technical summary §2 "Codificación de Pesos"]. Here the
// encoder is the same coder as the host encoder (range ANS, Duda 2013, with
// 64 interleaved states, Giesen 2014), run with one wavefront per chunk, and
// produces byte-identical regions.
//
// Mapping onto CDNA4: lane j of the wave owns rANS state j of the chunk and
// encodes the chunk's symbols i = 64 t + j, walking the steps t from last to
// first. Within a step the format's emission order is descending lane, so a
// lane's word position is the number of higher lanes that also emit
// (ballot + mbcnt, counted from the top); words fill the chunk's scratch
// area from its end towards its start, which leaves them in decoding order.
// Symbols reach the lanes through an LDS buffer filled 16 bytes per lane.
#include <hip/hip_runtime.h>

#include "entq.h"
#include "entq_internal.h"

namespace entq {
namespace {

constexpr int kEncWaves = 8;                 // chunks per workgroup
constexpr int kEncThreads = kEncWaves * 64;
constexpr uint32_t kEncStageSteps = 16;      // steps per symbol stage (1 KB)

// The table by value: freq and start of each byte (start = sum of the
// frequencies of the smaller bytes).
struct EncTable {
    uint16_t freq[256];
    uint16_t start[256];
};

__device__ __forceinline__ uint32_t lane_prefix_enc(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// floor(x / f) for x < 2^32, 1 <= f <= 4096, with recip = floor(2^44 / f) + 1:
// x * recip / 2^44 exceeds x / f by less than 2^-12 <= 1/f, and x / f is at
// most (f - 1) / f above its floor. The 96-bit product's bits 44.. are
// (x * (recip >> 32) + ((x * (recip & 0xFFFFFFFF)) >> 32)) >> 12.
__device__ __forceinline__ uint32_t div_by_freq(uint32_t x, uint64_t recip) {
    const uint64_t lo = (uint64_t)x * (uint32_t)recip;
    const uint64_t hi = (uint64_t)x * (uint32_t)(recip >> 32) + (lo >> 32);
    return (uint32_t)(hi >> 12);
}

// Scratch layout of one tensor: per chunk k, 64 u32 final states at
// k * stride, then room for chunk_symbols u16 words filled from the end.
__host__ __device__ inline uint64_t scratch_stride(uint32_t chunk_symbols) {
    return ((uint64_t)kStateBytes + 2ull * chunk_symbols + 15u) & ~(uint64_t)15u;
}

__global__ __launch_bounds__(kEncThreads) void encode_chunks(
    EncTable table, const uint8_t *__restrict__ symbols, uint64_t n, uint32_t chunk_symbols,
    uint64_t n_chunks, uint8_t *__restrict__ scratch, uint32_t *__restrict__ n_words_out) {
    __shared__ uint32_t F[256];       // f
    __shared__ uint32_t S[256];       // start
    __shared__ uint64_t R[256];       // floor(2^44 / f) + 1 (0 if f = 0)
    __shared__ __attribute__((aligned(16))) uint8_t STAGE[kEncWaves][64 * kEncStageSteps];

    for (uint32_t s = threadIdx.x; s < 256; s += kEncThreads) {
        const uint32_t f = table.freq[s];
        F[s] = f;
        S[s] = table.start[s];
        R[s] = f ? ((1ull << 44) / f) + 1 : 0;
    }
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t k = (uint64_t)blockIdx.x * kEncWaves + wave;
    if (k >= n_chunks) return;
    const uint64_t e0 = k * chunk_symbols;
    const uint32_t cn = (uint32_t)((n - e0 < chunk_symbols) ? n - e0 : chunk_symbols);
    const uint8_t *sym = symbols + e0;
    uint8_t *area = scratch + k * scratch_stride(chunk_symbols);
    uint16_t *words = reinterpret_cast<uint16_t *>(area + kStateBytes);
    uint8_t *stage = STAGE[wave];

    uint32_t x = kStateLow;
    uint32_t w = chunk_symbols;  // next word goes to words[w - 1]
    bool bad = false;            // a symbol with frequency 0
    const uint32_t steps = (cn + 63) / 64;
    // stages of kEncStageSteps steps, last stage first
    const uint32_t stages = (steps + kEncStageSteps - 1) / kEncStageSteps;
    for (uint32_t g = stages; g-- > 0;) {
        // lane l copies bytes [16 l, 16 l + 16) of the stage (inside the chunk)
        const uint32_t b0 = g * 64 * kEncStageSteps;
        const uint32_t b = b0 + 16u * lane;
        if (b + 16 <= cn) {
            *reinterpret_cast<uint4 *>(stage + 16u * lane) =
                *reinterpret_cast<const uint4 *>(sym + b);
        } else {
            for (uint32_t q = 0; q < 16; ++q)
                stage[16u * lane + q] = (b + q < cn) ? sym[b + q] : 0;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint32_t t1 = (g + 1) * kEncStageSteps < steps ? (g + 1) * kEncStageSteps : steps;
        for (uint32_t t = t1; t-- > g * kEncStageSteps;) {
            const uint32_t i = 64u * t + lane;
            const bool active = i < cn;
            const uint32_t s = stage[i - b0];
            const uint32_t f = F[s];
            // renormalise first: a state at or above 2^20 f sheds its low word
            // (f = 4096 never does: the bound is 2^32)
            const bool emit = active && f < kProbScale && x >= (f << 20);
            const uint64_t mask = __ballot(emit);
            const uint32_t cnt = (uint32_t)__popcll(mask);
            if (emit) {
                // emission order within a step is descending lane: the
                // higher emitting lanes' words come first (at higher indices)
                words[w - cnt + lane_prefix_enc(mask)] = (uint16_t)x;
                x >>= 16;
            }
            w -= cnt;
            if (active) {
                if (f == 0) {
                    bad = true;
                } else {
                    const uint32_t q = div_by_freq(x, R[s]);
                    x = (q << kProbBits) + (x - q * f) + S[s];
                }
            }
        }
        __builtin_amdgcn_wave_barrier();  // the stage is rewritten next
    }
    reinterpret_cast<uint32_t *>(area)[lane] = x;
    const uint64_t any_bad = __ballot(bad);
    if (lane == 0) n_words_out[k] = any_bad ? 0xFFFFFFFFu : chunk_symbols - w;
}

// One workgroup per chunk: region = 64 states, the words (the last n_words
// of the chunk's word area), zeros up to the next 16-byte boundary.
__global__ __launch_bounds__(256) void pack_chunks(const uint8_t *__restrict__ scratch,
                                                   uint32_t chunk_symbols,
                                                   const uint32_t *__restrict__ n_words,
                                                   const uint64_t *__restrict__ offsets,
                                                   uint8_t *__restrict__ blob) {
    const uint64_t k = blockIdx.x;
    const uint32_t nw = n_words[k];
    if (nw > chunk_symbols) return;  // a chunk the encoder rejected (frequency-0 symbol)
    const uint8_t *area = scratch + k * scratch_stride(chunk_symbols);
    const uint16_t *src = reinterpret_cast<const uint16_t *>(area + kStateBytes) + (chunk_symbols - nw);
    uint8_t *dst = blob + offsets[k];
    if (threadIdx.x < 64)
        reinterpret_cast<uint32_t *>(dst)[threadIdx.x] = reinterpret_cast<const uint32_t *>(area)[threadIdx.x];
    uint16_t *dw = reinterpret_cast<uint16_t *>(dst + kStateBytes);
    const uint32_t padded = (uint32_t)(((kStateBytes + 2ull * nw + 15u) & ~15ull) - kStateBytes) / 2;
    for (uint32_t i = threadIdx.x; i < padded; i += blockDim.x) dw[i] = (i < nw) ? src[i] : 0;
}

__global__ __launch_bounds__(256) void count_bytes(const uint8_t *__restrict__ symbols, uint64_t n,
                                                   unsigned long long *__restrict__ counts) {
    __shared__ uint32_t H[256];
    H[threadIdx.x] = 0;
    __syncthreads();
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 16;
    for (uint64_t b = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; b < n; b += stride) {
        if (b + 16 <= n) {
            const uint4 v = *reinterpret_cast<const uint4 *>(symbols + b);
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
            for (int q = 0; q < 4; ++q)
                for (int c = 0; c < 4; ++c) atomicAdd(&H[(u[q] >> (8 * c)) & 0xFFu], 1u);
        } else {
            for (uint64_t q = b; q < n; ++q) atomicAdd(&H[symbols[q]], 1u);
        }
    }
    __syncthreads();
    if (H[threadIdx.x]) atomicAdd(&counts[threadIdx.x], (unsigned long long)H[threadIdx.x]);
}

}  // namespace
}  // namespace entq

extern "C" {

entq_status entq_count_symbols_device(const uint8_t *d_symbols, uint64_t n, uint64_t *d_counts,
                                      void *stream) {
    if (!d_counts || (n && !d_symbols)) return ENTQ_EINVAL;
    if (n && (uintptr_t)d_symbols % 16) return ENTQ_EALIGN;
    if ((uintptr_t)d_counts % 8) return ENTQ_EALIGN;
    if (n == 0) return ENTQ_OK;
    uint64_t blocks = (n + 256 * 16 * 64 - 1) / (256 * 16 * 64);  // >= 64 bytes-per-thread rounds
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(entq::count_bytes, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, d_symbols, n,
                       reinterpret_cast<unsigned long long *>(d_counts));
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

uint64_t entq_region_bytes(uint32_t n_words) {
    return ((uint64_t)entq::kStateBytes + 2ull * n_words + (ENTQ_REGION_ALIGN - 1)) &
           ~(uint64_t)(ENTQ_REGION_ALIGN - 1);
}

uint64_t entq_encode_device_scratch_bytes(uint64_t n_symbols, uint32_t chunk_symbols) {
    if (chunk_symbols == 0) return 0;
    const uint64_t k = (n_symbols + chunk_symbols - 1) / chunk_symbols;
    return k * entq::scratch_stride(chunk_symbols);
}

entq_status entq_encode_device(const uint8_t *d_symbols, uint64_t n, uint32_t chunk_symbols,
                               const uint16_t freq[256], void *d_scratch, uint64_t scratch_bytes,
                               uint32_t *d_n_words, void *stream) {
    if (!freq || (n && (!d_symbols || !d_scratch || !d_n_words))) return ENTQ_EINVAL;
    if (chunk_symbols == 0 || chunk_symbols % entq::kLanes ||
        chunk_symbols > entq::kMaxChunkSymbols)
        return ENTQ_EINVAL;
    if (n == 0) return ENTQ_OK;
    if ((uintptr_t)d_symbols % 16 || (uintptr_t)d_scratch % 16 || (uintptr_t)d_n_words % 4)
        return ENTQ_EALIGN;
    if (scratch_bytes < entq_encode_device_scratch_bytes(n, chunk_symbols)) return ENTQ_EWORKSPACE;
    entq::EncTable table;
    uint32_t total = 0;
    for (int s = 0; s < 256; ++s) {
        table.freq[s] = freq[s];
        table.start[s] = (uint16_t)total;
        total += freq[s];
        if (freq[s] > entq::kProbScale) return ENTQ_EBADTABLE;
    }
    if (total != entq::kProbScale) return ENTQ_EBADTABLE;
    const uint64_t n_chunks = (n + chunk_symbols - 1) / chunk_symbols;
    const uint64_t blocks = (n_chunks + entq::kEncWaves - 1) / entq::kEncWaves;
    if (blocks > 0x7FFFFFFF) return ENTQ_EINVAL;
    hipLaunchKernelGGL(entq::encode_chunks, dim3((unsigned)blocks), dim3(entq::kEncThreads), 0,
                       (hipStream_t)stream, table, d_symbols, n, chunk_symbols, n_chunks,
                       static_cast<uint8_t *>(d_scratch), d_n_words);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

entq_status entq_pack_device(const void *d_scratch, uint64_t n, uint32_t chunk_symbols,
                             const uint32_t *d_n_words, const uint64_t *d_byte_offsets,
                             void *d_blob, void *stream) {
    if (chunk_symbols == 0 || chunk_symbols % entq::kLanes ||
        chunk_symbols > entq::kMaxChunkSymbols)
        return ENTQ_EINVAL;
    if (n == 0) return ENTQ_OK;
    if (!d_scratch || !d_n_words || !d_byte_offsets || !d_blob) return ENTQ_EINVAL;
    if ((uintptr_t)d_blob % ENTQ_REGION_ALIGN || (uintptr_t)d_scratch % 16) return ENTQ_EALIGN;
    const uint64_t n_chunks = (n + chunk_symbols - 1) / chunk_symbols;
    if (n_chunks > 0x7FFFFFFF) return ENTQ_EINVAL;
    hipLaunchKernelGGL(entq::pack_chunks, dim3((unsigned)n_chunks), dim3(256), 0,
                       (hipStream_t)stream, static_cast<const uint8_t *>(d_scratch),
                       chunk_symbols, d_n_words, d_byte_offsets, static_cast<uint8_t *>(d_blob));
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

}  // extern "C"

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

constexpr int kEncWaves = 4;                 // chunks per workgroup
constexpr int kEncThreads = kEncWaves * 64;
constexpr uint32_t kEncGroup = 8;            // steps whose symbols are loaded together
constexpr int kMaxEncJobs = 16;              // tensors per launch

// One encoding job (a tensor) as the kernel sees it. Its workgroups are
// first_block .. first_block + ceil(n_chunks / kEncWaves) - 1.
struct EncJob {
    const uint8_t *symbols;
    uint8_t *scratch;
    uint32_t *n_words;
    const uint16_t *freq;    // device table (batched calls)
    uint64_t n;
    uint32_t chunk_symbols;
    uint32_t n_chunks;
    uint32_t first_block;
    uint32_t pad;
};

struct EncJobs {
    EncJob job[kMaxEncJobs];
    uint32_t n_jobs;
};

// The host table of a single-tensor call, by value.
struct EncFreq {
    uint16_t f[256];
};

// Everything one encoding step needs about a symbol s with frequency f and
// cumulative start c, in one 32-byte LDS entry:
//   xmax_m1 = 2^20 f - 1: the state sheds a word when x > xmax_m1 (never
//             for f = 4096, whose bound 2^32 is out of range);
//   rcp     = 1/f rounded to the nearest fp32;
//   nf, f, g = -f, f, 4096 - f;
//   c       = c, with bit 31 set when f = 0 (such a symbol cannot be coded).
struct alignas(32) EncEntry {
    uint32_t xmax_m1;
    float rcp;
    int32_t nf;
    uint32_t f;
    uint32_t g;
    uint32_t c;
    uint32_t pad[2];
};

__device__ __forceinline__ EncEntry make_entry(uint32_t f, uint32_t c) {
    EncEntry e;
    e.xmax_m1 = (f == 0 || f >= kProbScale) ? 0xFFFFFFFFu : (f << 20) - 1u;
    e.rcp = f ? (float)(1.0 / (double)f) : 0.0f;
    e.nf = -(int32_t)f;
    e.f = f;
    e.g = kProbScale - f;
    e.c = f ? c : 0x80000000u;
    e.pad[0] = e.pad[1] = 0;
    return e;
}

__device__ __forceinline__ uint32_t lane_prefix_enc(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// The coding step x' = floor(x / f) 2^12 + (x mod f) + c = x + q (4096 - f)
// + c, q = floor(x / f), for a renormalised state (x < 2^20 f, so
// y = x / f < 2^20), with full-rate fp32 and 24-bit integer operations only.
// The estimate z = fl(fl(x) * fl(1/f) - 1/4) is within 2^-23 y + 2^-5 < 0.16
// of y - 1/4: each of the three roundings is relative 2^-24 or, for the
// last, half an ulp below 2^20. With y = q + r/f, 0 <= r <= f - 1, z lies in
// (q - 1, q + 1) and truncates to q - 1 or q (to 0 for q = 0); the remainder
// x - q_est f, in [0, 2f), tells which, and a short estimate adds one more
// 4096 - f. For f = 4096 (a single-symbol tensor) the step keeps x whatever
// q_est is, as 4096 - f = 0 and c = 0.
__device__ __forceinline__ uint32_t code_step(uint32_t x, const EncEntry &e) {
    const float z = __builtin_fmaf((float)x, e.rcp, -0.25f);
    const uint32_t q = (uint32_t)(int32_t)z;                     // z > -1
    const uint32_t r = x + (uint32_t)__mul24((int32_t)q, e.nf);  // x - q f, exact mod 2^32
    const uint32_t fix = r >= e.f ? e.g : 0u;
    return __umul24(q, e.g) + x + e.c + fix;
}

// Scratch layout of one tensor: per chunk k, 64 u32 final states at
// k * stride, then room for chunk_symbols u16 words filled from the end.
__host__ __device__ inline uint64_t scratch_stride(uint32_t chunk_symbols) {
    return ((uint64_t)kStateBytes + 2ull * chunk_symbols + 15u) & ~(uint64_t)15u;
}

// The symbols of steps 16 g .. 16 g + 15 for this lane. kGuard: the group
// may reach past the chunk's cn symbols (0 there); below the top group
// every step is full.
template <bool kGuard>
__device__ __forceinline__ void load_group(const uint8_t *__restrict__ sym, uint32_t cn,
                                           uint32_t g, uint32_t lane, uint32_t (&a)[kEncGroup]) {
#pragma unroll
    for (uint32_t k = 0; k < kEncGroup; ++k) {
        const uint32_t i = 64u * (kEncGroup * g + k) + lane;
        a[k] = (!kGuard || i < cn) ? sym[i] : 0u;
    }
}

// Waits until every vector memory operation of the wave has completed
// (s_waitcnt vmcnt(0); the other counters left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Codes the steps of group g, last first. The entry of the next step's
// symbol is read from LDS before the current step is coded, so the read
// overlaps the arithmetic. kTop: the group holding the chunk's last step,
// which may be partial (steps at or past `steps` skipped, lanes past cn
// inactive); every other group is full.
template <bool kTop>
__device__ __forceinline__ void code_group(const EncEntry *__restrict__ T,
                                           const uint32_t (&cur)[kEncGroup], uint32_t g,
                                           uint32_t steps, uint32_t cn, uint32_t lane,
                                           uint32_t &x, uint32_t &w, uint32_t &bad,
                                           uint16_t *__restrict__ words) {
    int k = kEncGroup - 1;
    if (kTop)
        while (k > 0 && kEncGroup * g + (uint32_t)k >= steps) --k;  // uniform
    EncEntry e = T[cur[k]];
#pragma unroll
    for (int kk = kEncGroup - 1; kk >= 0; --kk) {
        if (kTop && kk > k) continue;
        const uint32_t t = kEncGroup * g + (uint32_t)kk;
        const bool active = !kTop || 64u * t + lane < cn;
        const EncEntry en = T[cur[kk > 0 ? kk - 1 : 0]];  // next step's entry
        // renormalise first: a state above 2^20 f - 1 sheds its low word
        const bool emit = active && x > e.xmax_m1;
        const uint64_t mask = __ballot(emit);
        const uint32_t cnt = (uint32_t)__popcll(mask);
        // emission order within a step is descending lane: the higher
        // emitting lanes' words come first (at higher indices)
        w -= cnt;
        uint16_t *const wb = words + w;  // uniform base: the store takes a lane offset only
        if (emit) wb[lane_prefix_enc(mask)] = (uint16_t)x;
        const uint32_t xr = emit ? x >> 16 : x;
        const uint32_t xn = code_step(xr, e);
        x = active ? xn : xr;
        bad |= active ? e.c : 0u;
        e = en;
    }
}

// One wave encodes one chunk: cn symbols at sym, final states and words
// into area. Returns the word count, or 0xFFFFFFFF if a symbol has
// frequency 0. Steps run from last to first in groups of kEncGroup; the
// symbols of the next group are loaded while the current group is coded.
__device__ __forceinline__ uint32_t encode_chunk(const EncEntry *__restrict__ T,
                                                 const uint8_t *__restrict__ sym, uint32_t cn,
                                                 uint32_t chunk_symbols, uint8_t *__restrict__ area,
                                                 uint32_t lane) {
    uint16_t *words = reinterpret_cast<uint16_t *>(area + kStateBytes);
    uint32_t x = kStateLow;
    uint32_t w = chunk_symbols;  // next word goes to words[w - 1]
    uint32_t bad = 0;
    const uint32_t steps = (cn + 63) / 64;
    // two symbol buffers used in turn: one being coded, one being loaded
    uint32_t sa[kEncGroup], sb[kEncGroup];
    uint32_t g = (steps - 1) / kEncGroup;
    load_group<true>(sym, cn, g, lane, sa);
    wait_vmem();
    if (g > 0) load_group<false>(sym, cn, g - 1, lane, sb);
    code_group<true>(T, sa, g, steps, cn, lane, x, w, bad, words);
    while (g > 0) {
        --g;
        wait_vmem();  // this group's symbols (and earlier word stores)
        if (g > 0) load_group<false>(sym, cn, g - 1, lane, sa);
        code_group<false>(T, sb, g, steps, cn, lane, x, w, bad, words);
        if (g == 0) break;
        --g;
        wait_vmem();
        if (g > 0) load_group<false>(sym, cn, g - 1, lane, sb);
        code_group<false>(T, sa, g, steps, cn, lane, x, w, bad, words);
    }
    reinterpret_cast<uint32_t *>(area)[lane] = x;
    const uint64_t any_bad = __ballot(bad >> 31);
    return any_bad ? 0xFFFFFFFFu : chunk_symbols - w;
}

// Builds the 256 entries from a frequency table (read by threads 0..255;
// cumulative starts by a Hillis-Steele scan). Returns whether the table
// sums to 4096 with every f <= 4096.
__device__ bool build_entries(EncEntry *T, uint32_t *P, const uint16_t *freq) {
    const uint32_t s = threadIdx.x;
    const uint32_t f = s < 256 ? freq[s] : 0u;
    if (s < 256) P[s] = f;
    __syncthreads();
    for (uint32_t d = 1; d < 256; d <<= 1) {
        const uint32_t v = (s < 256 && s >= d) ? P[s - d] : 0u;
        __syncthreads();
        if (s < 256) P[s] += v;
        __syncthreads();
    }
    const uint32_t total = P[255];
    if (s < 256) T[s] = make_entry(f > kProbScale ? 0u : f, P[s] - f);
    const bool over = __syncthreads_or(s < 256 && f > kProbScale);
    return total == kProbScale && !over;
}

// The entries of one chunk's own table, built by one wave: lane l takes
// symbols 4l .. 4l+3, a wave scan gives the cumulative starts. Returns
// whether the table sums to 4096 with every f <= 4096.
__device__ bool build_entries_wave(EncEntry *T, const uint16_t *__restrict__ freq, uint32_t lane) {
    uint32_t f[4], pre[4], tot = 0;
    for (int i = 0; i < 4; ++i) {
        f[i] = freq[4u * lane + i];
        pre[i] = tot;
        tot += f[i];
    }
    uint32_t incl = tot;  // inclusive scan over lanes
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const uint32_t v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    const uint32_t start = incl - tot;
    bool over = false;
    for (int i = 0; i < 4; ++i) {
        over |= f[i] > kProbScale;
        T[4u * lane + i] = make_entry(f[i] > kProbScale ? 0u : f[i], start + pre[i]);
    }
    const uint32_t total = __shfl(incl, 63, 64);
    const bool any_over = __ballot(over) != 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return total == kProbScale && !any_over;
}

// Chunks that carry their own tables: job.freq holds one table per chunk
// (256 u16 each); each wave builds the entries of its chunk's table.
__global__ __launch_bounds__(kEncThreads) void encode_chunks_own_tables(EncJobs jobs) {
    __shared__ EncEntry TW[kEncWaves][256];
    uint32_t j = 0;
    while (j + 1 < jobs.n_jobs && jobs.job[j + 1].first_block <= blockIdx.x) ++j;
    const EncJob &job = jobs.job[j];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t k = (uint64_t)(blockIdx.x - job.first_block) * kEncWaves + wave;
    if (k >= job.n_chunks) return;
    if (!build_entries_wave(TW[wave], job.freq + k * 256, lane)) {
        if (lane == 0) job.n_words[k] = 0xFFFFFFFFu;
        return;
    }
    const uint64_t e0 = k * job.chunk_symbols;
    const uint32_t cn =
        (uint32_t)((job.n - e0 < job.chunk_symbols) ? job.n - e0 : job.chunk_symbols);
    const uint32_t nw = encode_chunk(TW[wave], job.symbols + e0, cn, job.chunk_symbols,
                                     job.scratch + k * scratch_stride(job.chunk_symbols), lane);
    if (lane == 0) job.n_words[k] = nw;
}

template <bool kInlineTable>
__global__ __launch_bounds__(kEncThreads) void encode_chunks(EncJobs jobs, EncFreq inline_freq) {
    __shared__ EncEntry T[256];
    __shared__ uint32_t P[256];
    uint32_t j = 0;
    while (j + 1 < jobs.n_jobs && jobs.job[j + 1].first_block <= blockIdx.x) ++j;
    const EncJob &job = jobs.job[j];
    const bool ok = build_entries(T, P, kInlineTable ? inline_freq.f : job.freq);
    __syncthreads();

    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t k = (uint64_t)(blockIdx.x - job.first_block) * kEncWaves + wave;
    if (k >= job.n_chunks) return;
    if (!ok) {
        if (lane == 0) job.n_words[k] = 0xFFFFFFFFu;
        return;
    }
    const uint64_t e0 = k * job.chunk_symbols;
    const uint32_t cn =
        (uint32_t)((job.n - e0 < job.chunk_symbols) ? job.n - e0 : job.chunk_symbols);
    const uint32_t nw = encode_chunk(T, job.symbols + e0, cn, job.chunk_symbols,
                                     job.scratch + k * scratch_stride(job.chunk_symbols), lane);
    if (lane == 0) job.n_words[k] = nw;
}

// One workgroup per chunk: region = 64 states, the words (the last n_words
// of the chunk's word area), zeros up to the next 16-byte boundary. The
// region is written one dword per thread and pass; when the words start at
// an odd word index, each dword is funnelled from two source dwords.
// With own_tables (one u16 table of 256 per chunk) the region starts with the
// chunk's table, ENTQ_TABLE_BYTES, before the states.
__device__ __forceinline__ void pack_one(const uint8_t *__restrict__ scratch,
                                         uint32_t chunk_symbols,
                                         const uint32_t *__restrict__ n_words,
                                         const uint64_t *__restrict__ offsets,
                                         uint8_t *__restrict__ blob, uint64_t k,
                                         const uint16_t *__restrict__ own_tables = nullptr) {
    const uint32_t nw = n_words[k];
    if (nw > chunk_symbols) return;  // a chunk the encoder rejected (frequency-0 symbol)
    const uint8_t *area = scratch + k * scratch_stride(chunk_symbols);
    uint32_t *dst = reinterpret_cast<uint32_t *>(blob + offsets[k]);
    if (own_tables) {
        const uint32_t *tab = reinterpret_cast<const uint32_t *>(own_tables + k * 256);
        if (threadIdx.x < ENTQ_TABLE_BYTES / 4) dst[threadIdx.x] = tab[threadIdx.x];
        dst += ENTQ_TABLE_BYTES / 4;
    }
    if (threadIdx.x < 64) dst[threadIdx.x] = reinterpret_cast<const uint32_t *>(area)[threadIdx.x];
    const uint32_t *A = reinterpret_cast<const uint32_t *>(area + kStateBytes);  // word pairs
    uint32_t *D = dst + kStateBytes / 4;
    const uint32_t sb = chunk_symbols - nw;  // first word
    const uint32_t n_dw = (uint32_t)((((uint64_t)kStateBytes + 2ull * nw + 15u) & ~15ull) -
                                     kStateBytes) / 4;  // dwords after the states
    const uint32_t full = nw / 2;                       // dwords holding two words
    if ((sb & 1u) == 0) {
        const uint32_t a0 = sb / 2;
        for (uint32_t d = threadIdx.x; d < n_dw; d += 256) {
            uint32_t v = 0;
            if (d < full) v = A[a0 + d];
            else if (d == full && (nw & 1u)) v = A[a0 + d] & 0xFFFFu;
            D[d] = v;
        }
    } else {
        // word sb + 2d sits in the high half of dword (sb - 1) / 2 + d
        const uint32_t a0 = (sb - 1) / 2;
        for (uint32_t d = threadIdx.x; d < n_dw; d += 256) {
            uint32_t v = 0;
            if (d < full) {
                v = __builtin_amdgcn_alignbit(A[a0 + d + 1], A[a0 + d], 16);
            } else if (d == full && (nw & 1u)) {
                v = A[a0 + d] >> 16;
            }
            D[d] = v;
        }
    }
}

__global__ __launch_bounds__(256) void pack_chunks(const uint8_t *__restrict__ scratch,
                                                   uint32_t chunk_symbols,
                                                   const uint32_t *__restrict__ n_words,
                                                   const uint64_t *__restrict__ offsets,
                                                   uint8_t *__restrict__ blob) {
    pack_one(scratch, chunk_symbols, n_words, offsets, blob, blockIdx.x);
}

// Several tensors in one launch (one blob): job j packs its chunks with
// workgroups first_block .. first_block + n_chunks - 1.
struct PackJob {
    const uint8_t *scratch;
    const uint32_t *n_words;
    const uint64_t *offsets;
    const uint16_t *own_tables;  // per-chunk tables, or null
    uint32_t chunk_symbols, first_block;
};
struct PackJobs {
    PackJob job[kMaxEncJobs];
    uint32_t n_jobs;
};

__global__ __launch_bounds__(256) void pack_chunks_batch(PackJobs jobs, uint8_t *__restrict__ blob) {
    uint32_t j = 0;
    while (j + 1 < jobs.n_jobs && jobs.job[j + 1].first_block <= blockIdx.x) ++j;
    const PackJob &pj = jobs.job[j];
    pack_one(pj.scratch, pj.chunk_symbols, pj.n_words, pj.offsets, blob,
             blockIdx.x - pj.first_block, pj.own_tables);
}

// Region offsets: offsets[k] = base + the region bytes of chunks 0..k-1
// (256 + 2 n_words rounded up to 16; a chunk marked rejected, n_words above
// any chunk size, takes none), *end = base + all of them. One workgroup:
// each thread sums a run of consecutive chunks, a Hillis-Steele scan over
// the 1024 run sums gives each run its start, the run is then written out.
constexpr int kScanThreads = 1024;

__device__ __forceinline__ uint64_t region_size(uint32_t nw, uint32_t header) {
    return nw > (uint32_t)kMaxChunkSymbols
               ? 0
               : header + (((uint64_t)kStateBytes + 2ull * nw + 15u) & ~15ull);
}

// header: bytes before the states of every region (0, or ENTQ_TABLE_BYTES
// for chunks that carry their own tables).
__global__ __launch_bounds__(kScanThreads) void region_offsets(const uint32_t *__restrict__ n_words,
                                                               uint64_t n_chunks, uint64_t base,
                                                               uint32_t header,
                                                               uint64_t *__restrict__ offsets,
                                                               uint64_t *__restrict__ end) {
    __shared__ uint64_t part[kScanThreads];
    const uint32_t t = threadIdx.x;
    const uint64_t per = (n_chunks + kScanThreads - 1) / kScanThreads;
    const uint64_t lo = t * per < n_chunks ? t * per : n_chunks;
    const uint64_t hi = lo + per < n_chunks ? lo + per : n_chunks;
    uint64_t sum = 0;
    for (uint64_t i = lo; i < hi; ++i) sum += region_size(n_words[i], header);
    part[t] = sum;
    __syncthreads();
    for (uint32_t d = 1; d < kScanThreads; d <<= 1) {
        const uint64_t v = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    uint64_t run = base + part[t] - sum;  // exclusive prefix of this run
    for (uint64_t i = lo; i < hi; ++i) {
        offsets[i] = run;
        run += region_size(n_words[i], header);
    }
    if (t == kScanThreads - 1) *end = base + part[t];
}

// Byte histogram. Each workgroup keeps one LDS table of 256 bins x 64 lane
// columns (64 KB): lane j adds into column j, so the 64 atomic adds of one
// wave instruction always fall into 64 different banks, however skewed the
// bytes are (a shared 256-bin table serialises the many lanes that hold the
// same common byte). The waves of the workgroup share the columns through the
// LDS atomics. Each lane reads 64 bytes per round as four 16-byte loads.
constexpr int kCountThreads = 512;
constexpr int kCountBytesPerLane = 64;

// The histogram of one workgroup's share of a byte array, left in H (bin b
// = the sum of row b's 64 columns): block bid of nblocks takes lane rounds
// bid * kCountThreads + t, + nblocks * kCountThreads, ...; block 0 also takes
// the last n % 64 bytes.
__device__ __forceinline__ void histogram(uint32_t *H, const uint8_t *__restrict__ symbols,
                                          uint64_t n, uint64_t bid, uint64_t nblocks) {
    const uint32_t lane_off = (threadIdx.x & 63u) * 4u;  // byte offset of the lane's column
    for (uint32_t i = threadIdx.x; i < 256u * 64u / 4u; i += kCountThreads)
        reinterpret_cast<uint4 *>(H)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    char *const Hb = reinterpret_cast<char *>(H);
    auto add_byte = [&](uint32_t b) {  // b < 256
        __hip_atomic_fetch_add(reinterpret_cast<uint32_t *>(Hb + ((b << 8) | lane_off)), 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto add4 = [&](uint32_t u) {
        for (int c = 0; c < 4; ++c) add_byte((u >> (8 * c)) & 0xFFu);
    };
    const uint64_t n_full = n / kCountBytesPerLane;  // whole 64-byte lane rounds
    const uint64_t stride = nblocks * kCountThreads;
    for (uint64_t r = bid * kCountThreads + threadIdx.x; r < n_full; r += stride) {
        const uint4 *src = reinterpret_cast<const uint4 *>(symbols + r * kCountBytesPerLane);
        uint4 v[4];
        for (int q = 0; q < 4; ++q) v[q] = src[q];
        for (int q = 0; q < 4; ++q) {
            add4(v[q].x);
            add4(v[q].y);
            add4(v[q].z);
            add4(v[q].w);
        }
    }
    // the last n % 64 bytes, one per thread of the first workgroup
    if (bid == 0) {
        const uint64_t tail = n_full * kCountBytesPerLane + threadIdx.x;
        if (tail < n) add_byte(symbols[tail]);
    }
    __syncthreads();
}

// Bin b of the histogram in H (thread b < 256).
__device__ __forceinline__ uint64_t histogram_bin(const uint32_t *H, uint32_t b) {
    uint64_t sum = 0;
    for (uint32_t j = 0; j < 64; ++j)  // column order rotated by bin: no bank conflicts
        sum += H[b * 64u + ((j + b) & 63u)];
    return sum;
}

// A workgroup's share added into 64-bit counts.
__device__ __forceinline__ void count_share(uint32_t *H, const uint8_t *__restrict__ symbols,
                                            uint64_t n, unsigned long long *__restrict__ counts,
                                            uint64_t bid, uint64_t nblocks) {
    histogram(H, symbols, n, bid, nblocks);
    if (threadIdx.x < 256) {
        const uint64_t sum = histogram_bin(H, threadIdx.x);
        if (sum) atomicAdd(&counts[threadIdx.x], (unsigned long long)sum);
    }
}

__global__ __launch_bounds__(kCountThreads) void count_bytes(const uint8_t *__restrict__ symbols,
                                                             uint64_t n,
                                                             unsigned long long *__restrict__ counts) {
    __shared__ uint32_t H[256 * 64];
    count_share(H, symbols, n, counts, blockIdx.x, gridDim.x);
}

// Several arrays in one launch: job j owns workgroups first_block ..
// first_block + blocks - 1.
struct CountJob {
    const uint8_t *symbols;
    unsigned long long *counts;
    uint64_t n;
    uint32_t first_block, blocks;
};
struct CountJobs {
    CountJob job[kMaxEncJobs];
    uint32_t n_jobs;
};

__global__ __launch_bounds__(kCountThreads) void count_bytes_batch(CountJobs jobs) {
    __shared__ uint32_t H[256 * 64];
    uint32_t j = 0;
    while (j + 1 < jobs.n_jobs && jobs.job[j + 1].first_block <= blockIdx.x) ++j;
    const CountJob &cj = jobs.job[j];
    count_share(H, cj.symbols, cj.n, cj.counts, blockIdx.x - cj.first_block, cj.blocks);
}

// Counts of every chunk of several arrays in one launch, one workgroup per
// chunk: job j's chunk k goes to counts[256 k ..] (32-bit: a chunk holds at
// most 2^20 bytes).
struct ChunkCountJob {
    const uint8_t *symbols;
    uint32_t *counts;
    uint64_t n;
    uint32_t chunk_symbols, first_block;
};
struct ChunkCountJobs {
    ChunkCountJob job[kMaxEncJobs];
    uint32_t n_jobs;
};

__global__ __launch_bounds__(kCountThreads) void count_chunks_batch(ChunkCountJobs jobs) {
    __shared__ uint32_t H[256 * 64];
    uint32_t j = 0;
    while (j + 1 < jobs.n_jobs && jobs.job[j + 1].first_block <= blockIdx.x) ++j;
    const ChunkCountJob &cj = jobs.job[j];
    const uint64_t k = blockIdx.x - cj.first_block;
    const uint64_t e0 = k * cj.chunk_symbols;
    const uint64_t cn = (cj.n - e0 < cj.chunk_symbols) ? cj.n - e0 : cj.chunk_symbols;
    histogram(H, cj.symbols + e0, cn, 0, 1);
    if (threadIdx.x < 256) cj.counts[k * 256 + threadIdx.x] = (uint32_t)histogram_bin(H, threadIdx.x);
}

// ---- tables from counts on the device --------------------------------------
//
// The table rule of entq_build_freq, one wave per table (lane l holds bytes
// 4l .. 4l+3): nearest share of 4096 (halves up), at least 1 for a present
// byte; a surplus is taken from the largest shares, smallest byte first on
// ties, and a shortfall given to the most frequent byte (smallest on ties);
// one present byte gets 4096, none gives an all-zero table. Taking one unit
// at a time from the current largest share is done in one pass: every share
// is capped at the smallest level L whose cap costs at most the surplus K,
// and the K - cost(L) units left come off the smallest bytes standing at L.

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

__device__ __forceinline__ uint32_t wave_sum32(uint32_t v) {
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

template <typename CountT>
__device__ void build_table_wave(const CountT *__restrict__ counts, uint16_t *__restrict__ freq,
                                 uint32_t lane) {
    uint64_t c[4];
    uint64_t n_loc = 0;
    uint32_t p_loc = 0;
    for (int i = 0; i < 4; ++i) {
        c[i] = counts[4u * lane + i];
        n_loc += c[i];
        p_loc += c[i] ? 1u : 0u;
    }
    const uint64_t N = wave_sum64(n_loc);
    const uint32_t present = wave_sum32(p_loc);
    uint32_t q[4] = {0, 0, 0, 0};
    if (present == 1) {
        for (int i = 0; i < 4; ++i) q[i] = c[i] ? kProbScale : 0u;
    } else if (present > 1) {
        uint32_t s_loc = 0;
        for (int i = 0; i < 4; ++i) {
            if (c[i]) {
                const uint64_t v = (2ull * kProbScale * c[i] + N) / (2ull * N);
                q[i] = v < 1 ? 1u : (uint32_t)v;
            }
            s_loc += q[i];
        }
        const uint32_t sum = wave_sum32(s_loc);
        if (sum > kProbScale) {
            const uint32_t K = sum - kProbScale;
            auto cost = [&](uint32_t L) {
                uint32_t d = 0;
                for (int i = 0; i < 4; ++i) d += q[i] > L ? q[i] - L : 0u;
                return wave_sum32(d);
            };
            uint32_t lo = 1, hi = kProbScale;  // smallest L with cost(L) <= K
            while (lo < hi) {
                const uint32_t mid = (lo + hi) / 2;
                if (cost(mid) <= K) hi = mid;
                else lo = mid + 1;
            }
            const uint32_t L = lo;
            const uint32_t r = K - cost(L);
            uint32_t at_loc = 0;
            for (int i = 0; i < 4; ++i) at_loc += q[i] >= L ? 1u : 0u;
            uint32_t incl = at_loc;  // bytes at level L up to this lane
            for (uint32_t d = 1; d < 64; d <<= 1) {
                const uint32_t v = __shfl_up(incl, d, 64);
                if (lane >= d) incl += v;
            }
            uint32_t rank = incl - at_loc;
            for (int i = 0; i < 4; ++i) {
                if (q[i] >= L) {
                    q[i] = (rank < r) ? L - 1 : L;
                    ++rank;
                }
            }
        } else if (sum < kProbScale) {
            // most frequent byte, smallest on ties
            uint64_t best = c[0];
            uint32_t arg = 4u * lane;
            for (int i = 1; i < 4; ++i)
                if (c[i] > best) { best = c[i]; arg = 4u * lane + i; }
            for (int d = 32; d >= 1; d >>= 1) {
                const uint64_t ob = __shfl_xor(best, d, 64);
                const uint32_t oa = __shfl_xor(arg, d, 64);
                if (ob > best || (ob == best && oa < arg)) { best = ob; arg = oa; }
            }
            if ((arg >> 2) == lane) q[arg & 3u] += kProbScale - sum;
        }
    }
    for (int i = 0; i < 4; ++i) freq[4u * lane + i] = (uint16_t)q[i];
}

template <typename CountT>
__global__ __launch_bounds__(256) void build_tables(const CountT *__restrict__ counts,
                                                    uint64_t n_tables, uint16_t *__restrict__ freq) {
    const uint64_t t = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n_tables) return;
    build_table_wave(counts + t * 256, freq + t * 256, threadIdx.x & 63);
}

// Workgroups for counting n bytes: two per CU on 256 CUs at most, fewer for
// small inputs (at least 16 lane rounds per thread); a lane column counts at
// most n / (64 blocks) bytes, more blocks keep that below 2^32.
inline uint64_t count_blocks(uint64_t n) {
    const uint64_t rounds = n / kCountBytesPerLane;
    uint64_t blocks = (rounds + 16ull * kCountThreads - 1) / (16ull * kCountThreads);
    if (blocks > 512) blocks = 512;
    const uint64_t min_blocks = (n >> 37) + 1;
    return blocks < min_blocks ? min_blocks : blocks;
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
    const uint64_t blocks = entq::count_blocks(n);
    if (blocks > 0x7FFFFFFF) return ENTQ_EINVAL;
    hipLaunchKernelGGL(entq::count_bytes, dim3((unsigned)blocks), dim3(entq::kCountThreads), 0,
                       (hipStream_t)stream, d_symbols, n,
                       reinterpret_cast<unsigned long long *>(d_counts));
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

entq_status entq_count_symbols_device_batch(const entq_count_job *jobs, int n_jobs,
                                            void *stream) {
    if (n_jobs < 0 || (n_jobs && !jobs)) return ENTQ_EINVAL;
    for (int j = 0; j < n_jobs; ++j) {
        if (!jobs[j].d_counts || (jobs[j].n_symbols && !jobs[j].d_symbols)) return ENTQ_EINVAL;
        if ((jobs[j].n_symbols && (uintptr_t)jobs[j].d_symbols % 16) ||
            (uintptr_t)jobs[j].d_counts % 8)
            return ENTQ_EALIGN;
    }
    entq::CountJobs batch = {};
    uint64_t blocks = 0;
    auto flush = [&]() -> bool {
        if (batch.n_jobs == 0) return true;
        hipLaunchKernelGGL(entq::count_bytes_batch, dim3((unsigned)blocks),
                           dim3(entq::kCountThreads), 0, (hipStream_t)stream, batch);
        batch = {};
        blocks = 0;
        return hipGetLastError() == hipSuccess;
    };
    for (int j = 0; j < n_jobs; ++j) {
        if (jobs[j].n_symbols == 0) continue;
        const uint64_t b = entq::count_blocks(jobs[j].n_symbols);
        if (batch.n_jobs == (uint32_t)entq::kMaxEncJobs || blocks + b > 0x7FFFFFFFull)
            if (!flush()) return ENTQ_EHIP;
        batch.job[batch.n_jobs++] = {jobs[j].d_symbols,
                                     reinterpret_cast<unsigned long long *>(jobs[j].d_counts),
                                     jobs[j].n_symbols, (uint32_t)blocks, (uint32_t)b};
        blocks += b;
    }
    return flush() ? ENTQ_OK : ENTQ_EHIP;
}

entq_status entq_pack_device_batch(const entq_pack_job *jobs, int n_jobs, void *d_blob,
                                   void *stream) {
    if (n_jobs < 0 || (n_jobs && !jobs)) return ENTQ_EINVAL;
    if (n_jobs && !d_blob) return ENTQ_EINVAL;
    if ((uintptr_t)d_blob % ENTQ_REGION_ALIGN) return ENTQ_EALIGN;
    for (int j = 0; j < n_jobs; ++j) {
        const entq_pack_job &pj = jobs[j];
        const uint32_t C = pj.chunk_symbols;
        if (C == 0 || C % entq::kLanes || C > entq::kMaxChunkSymbols) return ENTQ_EINVAL;
        if (pj.n_symbols == 0) continue;
        if (!pj.d_scratch || !pj.d_n_words || !pj.d_byte_offsets) return ENTQ_EINVAL;
        if ((uintptr_t)pj.d_scratch % 16 || (uintptr_t)pj.d_n_words % 4 ||
            (uintptr_t)pj.d_byte_offsets % 8)
            return ENTQ_EALIGN;
        if ((pj.n_symbols + C - 1) / C > 0x7FFFFFFFull) return ENTQ_EINVAL;
    }
    entq::PackJobs batch = {};
    uint64_t blocks = 0;
    auto flush = [&]() -> bool {
        if (batch.n_jobs == 0) return true;
        hipLaunchKernelGGL(entq::pack_chunks_batch, dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, batch, static_cast<uint8_t *>(d_blob));
        batch = {};
        blocks = 0;
        return hipGetLastError() == hipSuccess;
    };
    for (int j = 0; j < n_jobs; ++j) {
        const entq_pack_job &pj = jobs[j];
        if (pj.n_symbols == 0) continue;
        const uint64_t k = (pj.n_symbols + pj.chunk_symbols - 1) / pj.chunk_symbols;
        if (batch.n_jobs == (uint32_t)entq::kMaxEncJobs || blocks + k > 0x7FFFFFFFull)
            if (!flush()) return ENTQ_EHIP;
        batch.job[batch.n_jobs++] = {static_cast<const uint8_t *>(pj.d_scratch), pj.d_n_words,
                                     pj.d_byte_offsets, nullptr, pj.chunk_symbols,
                                     (uint32_t)blocks};
        blocks += k;
    }
    return flush() ? ENTQ_OK : ENTQ_EHIP;
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
    uint32_t total = 0;
    for (int s = 0; s < 256; ++s) {
        if (freq[s] > entq::kProbScale) return ENTQ_EBADTABLE;
        total += freq[s];
    }
    if (total != entq::kProbScale) return ENTQ_EBADTABLE;
    if (n == 0) return ENTQ_OK;
    if ((uintptr_t)d_symbols % 16 || (uintptr_t)d_scratch % 16 || (uintptr_t)d_n_words % 4)
        return ENTQ_EALIGN;
    if (scratch_bytes < entq_encode_device_scratch_bytes(n, chunk_symbols)) return ENTQ_EWORKSPACE;
    const uint64_t n_chunks = (n + chunk_symbols - 1) / chunk_symbols;
    const uint64_t blocks = (n_chunks + entq::kEncWaves - 1) / entq::kEncWaves;
    if (blocks > 0x7FFFFFFF) return ENTQ_EINVAL;
    entq::EncJobs jobs = {};
    jobs.n_jobs = 1;
    jobs.job[0] = {d_symbols, static_cast<uint8_t *>(d_scratch), d_n_words, nullptr, n,
                   chunk_symbols, (uint32_t)n_chunks, 0, 0};
    entq::EncFreq table;
    for (int s = 0; s < 256; ++s) table.f[s] = freq[s];
    hipLaunchKernelGGL(entq::encode_chunks<true>, dim3((unsigned)blocks),
                       dim3(entq::kEncThreads), 0, (hipStream_t)stream, jobs, table);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

entq_status entq_encode_device_batch(const entq_encode_job *jobs, int n_jobs, void *stream) {
    if (n_jobs < 0 || (n_jobs && !jobs)) return ENTQ_EINVAL;
    for (int j = 0; j < n_jobs; ++j) {
        const entq_encode_job &jb = jobs[j];
        const uint32_t C = jb.chunk_symbols;
        if (C == 0 || C % entq::kLanes || C > entq::kMaxChunkSymbols) return ENTQ_EINVAL;
        if (jb.n_symbols == 0) continue;
        if (!jb.d_symbols || !jb.d_freq || !jb.d_scratch || !jb.d_n_words) return ENTQ_EINVAL;
        if ((uintptr_t)jb.d_symbols % 16 || (uintptr_t)jb.d_scratch % 16 ||
            (uintptr_t)jb.d_n_words % 4 || (uintptr_t)jb.d_freq % 2)
            return ENTQ_EALIGN;
        if (jb.scratch_bytes < entq_encode_device_scratch_bytes(jb.n_symbols, C))
            return ENTQ_EWORKSPACE;
        if ((jb.n_symbols + C - 1) / C > 0x7FFFFFFFull) return ENTQ_EINVAL;
    }
    // up to kMaxEncJobs non-empty jobs per launch, their workgroups back to back
    entq::EncJobs batch = {};
    uint64_t blocks = 0;
    const entq::EncFreq no_table = {};
    auto flush = [&]() -> bool {
        if (batch.n_jobs == 0) return true;
        hipLaunchKernelGGL(entq::encode_chunks<false>, dim3((unsigned)blocks),
                           dim3(entq::kEncThreads), 0, (hipStream_t)stream, batch, no_table);
        batch = {};
        blocks = 0;
        return hipGetLastError() == hipSuccess;
    };
    for (int j = 0; j < n_jobs; ++j) {
        const entq_encode_job &jb = jobs[j];
        if (jb.n_symbols == 0) continue;
        const uint64_t k = (jb.n_symbols + jb.chunk_symbols - 1) / jb.chunk_symbols;
        const uint64_t b = (k + entq::kEncWaves - 1) / entq::kEncWaves;
        if (batch.n_jobs == (uint32_t)entq::kMaxEncJobs || blocks + b > 0x7FFFFFFFull)
            if (!flush()) return ENTQ_EHIP;
        batch.job[batch.n_jobs++] = {jb.d_symbols, static_cast<uint8_t *>(jb.d_scratch),
                                     jb.d_n_words, jb.d_freq, jb.n_symbols, jb.chunk_symbols,
                                     (uint32_t)k, (uint32_t)blocks, 0};
        blocks += b;
    }
    return flush() ? ENTQ_OK : ENTQ_EHIP;
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

entq_status entq_region_offsets_device(const uint32_t *d_n_words, uint64_t n_chunks,
                                      uint64_t base_offset, uint64_t *d_byte_offsets,
                                      uint64_t *d_end_offset, void *stream) {
    if (!d_end_offset || (n_chunks && (!d_n_words || !d_byte_offsets))) return ENTQ_EINVAL;
    if ((uintptr_t)d_n_words % 4 || (uintptr_t)d_byte_offsets % 8 || (uintptr_t)d_end_offset % 8)
        return ENTQ_EALIGN;
    if (base_offset % ENTQ_REGION_ALIGN) return ENTQ_EALIGN;
    hipLaunchKernelGGL(entq::region_offsets, dim3(1), dim3(entq::kScanThreads), 0,
                       (hipStream_t)stream, d_n_words, n_chunks, base_offset, 0u,
                       d_byte_offsets, d_end_offset);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

entq_status entq_region_offsets_device_adaptive(const uint32_t *d_n_words, uint64_t n_chunks,
                                               uint64_t base_offset, uint64_t *d_byte_offsets,
                                               uint64_t *d_end_offset, void *stream) {
    if (!d_end_offset || (n_chunks && (!d_n_words || !d_byte_offsets))) return ENTQ_EINVAL;
    if ((uintptr_t)d_n_words % 4 || (uintptr_t)d_byte_offsets % 8 || (uintptr_t)d_end_offset % 8)
        return ENTQ_EALIGN;
    if (base_offset % ENTQ_REGION_ALIGN) return ENTQ_EALIGN;
    hipLaunchKernelGGL(entq::region_offsets, dim3(1), dim3(entq::kScanThreads), 0,
                       (hipStream_t)stream, d_n_words, n_chunks, base_offset,
                       (uint32_t)ENTQ_TABLE_BYTES, d_byte_offsets, d_end_offset);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

entq_status entq_build_freq_device(const void *d_counts, uint32_t count_bytes, uint64_t n_tables,
                                   uint16_t *d_freq, void *stream) {
    if (count_bytes != 4 && count_bytes != 8) return ENTQ_EINVAL;
    if (n_tables == 0) return ENTQ_OK;
    if (!d_counts || !d_freq) return ENTQ_EINVAL;
    if ((uintptr_t)d_counts % count_bytes || (uintptr_t)d_freq % 2) return ENTQ_EALIGN;
    const uint64_t blocks = (n_tables + 3) / 4;
    if (blocks > 0x7FFFFFFFull) return ENTQ_EINVAL;
    if (count_bytes == 4)
        hipLaunchKernelGGL(entq::build_tables<uint32_t>, dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, static_cast<const uint32_t *>(d_counts), n_tables,
                           d_freq);
    else
        hipLaunchKernelGGL(entq::build_tables<uint64_t>, dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, static_cast<const uint64_t *>(d_counts), n_tables,
                           d_freq);
    return hipGetLastError() == hipSuccess ? ENTQ_OK : ENTQ_EHIP;
}

entq_status entq_count_chunks_device_batch(const entq_chunk_count_job *jobs, int n_jobs,
                                           void *stream) {
    if (n_jobs < 0 || (n_jobs && !jobs)) return ENTQ_EINVAL;
    for (int j = 0; j < n_jobs; ++j) {
        const entq_chunk_count_job &cj = jobs[j];
        const uint32_t C = cj.chunk_symbols;
        if (C == 0 || C % entq::kLanes || C > entq::kMaxChunkSymbols) return ENTQ_EINVAL;
        if (cj.n_symbols == 0) continue;
        if (!cj.d_symbols || !cj.d_counts) return ENTQ_EINVAL;
        if ((uintptr_t)cj.d_symbols % 16 || (uintptr_t)cj.d_counts % 4) return ENTQ_EALIGN;
        if ((cj.n_symbols + C - 1) / C > 0x7FFFFFFFull) return ENTQ_EINVAL;
    }
    entq::ChunkCountJobs batch = {};
    uint64_t blocks = 0;
    auto flush = [&]() -> bool {
        if (batch.n_jobs == 0) return true;
        hipLaunchKernelGGL(entq::count_chunks_batch, dim3((unsigned)blocks),
                           dim3(entq::kCountThreads), 0, (hipStream_t)stream, batch);
        batch = {};
        blocks = 0;
        return hipGetLastError() == hipSuccess;
    };
    for (int j = 0; j < n_jobs; ++j) {
        const entq_chunk_count_job &cj = jobs[j];
        if (cj.n_symbols == 0) continue;
        const uint64_t k = (cj.n_symbols + cj.chunk_symbols - 1) / cj.chunk_symbols;
        if (batch.n_jobs == (uint32_t)entq::kMaxEncJobs || blocks + k > 0x7FFFFFFFull)
            if (!flush()) return ENTQ_EHIP;
        batch.job[batch.n_jobs++] = {cj.d_symbols, cj.d_counts, cj.n_symbols, cj.chunk_symbols,
                                     (uint32_t)blocks};
        blocks += k;
    }
    return flush() ? ENTQ_OK : ENTQ_EHIP;
}

entq_status entq_encode_device_adaptive_batch(const entq_encode_job *jobs, int n_jobs,
                                              void *stream) {
    if (n_jobs < 0 || (n_jobs && !jobs)) return ENTQ_EINVAL;
    for (int j = 0; j < n_jobs; ++j) {
        const entq_encode_job &jb = jobs[j];
        const uint32_t C = jb.chunk_symbols;
        if (C == 0 || C % entq::kLanes || C > entq::kMaxChunkSymbols) return ENTQ_EINVAL;
        if (jb.n_symbols == 0) continue;
        if (!jb.d_symbols || !jb.d_freq || !jb.d_scratch || !jb.d_n_words) return ENTQ_EINVAL;
        if ((uintptr_t)jb.d_symbols % 16 || (uintptr_t)jb.d_scratch % 16 ||
            (uintptr_t)jb.d_n_words % 4 || (uintptr_t)jb.d_freq % 2)
            return ENTQ_EALIGN;
        if (jb.scratch_bytes < entq_encode_device_scratch_bytes(jb.n_symbols, C))
            return ENTQ_EWORKSPACE;
        if ((jb.n_symbols + C - 1) / C > 0x7FFFFFFFull) return ENTQ_EINVAL;
    }
    entq::EncJobs batch = {};
    uint64_t blocks = 0;
    auto flush = [&]() -> bool {
        if (batch.n_jobs == 0) return true;
        hipLaunchKernelGGL(entq::encode_chunks_own_tables, dim3((unsigned)blocks),
                           dim3(entq::kEncThreads), 0, (hipStream_t)stream, batch);
        batch = {};
        blocks = 0;
        return hipGetLastError() == hipSuccess;
    };
    for (int j = 0; j < n_jobs; ++j) {
        const entq_encode_job &jb = jobs[j];
        if (jb.n_symbols == 0) continue;
        const uint64_t k = (jb.n_symbols + jb.chunk_symbols - 1) / jb.chunk_symbols;
        const uint64_t b = (k + entq::kEncWaves - 1) / entq::kEncWaves;
        if (batch.n_jobs == (uint32_t)entq::kMaxEncJobs || blocks + b > 0x7FFFFFFFull)
            if (!flush()) return ENTQ_EHIP;
        batch.job[batch.n_jobs++] = {jb.d_symbols, static_cast<uint8_t *>(jb.d_scratch),
                                     jb.d_n_words, jb.d_freq, jb.n_symbols, jb.chunk_symbols,
                                     (uint32_t)k, (uint32_t)blocks, 0};
        blocks += b;
    }
    return flush() ? ENTQ_OK : ENTQ_EHIP;
}

entq_status entq_pack_device_adaptive_batch(const entq_pack_adaptive_job *jobs, int n_jobs,
                                            void *d_blob, void *stream) {
    if (n_jobs < 0 || (n_jobs && !jobs)) return ENTQ_EINVAL;
    if (n_jobs && !d_blob) return ENTQ_EINVAL;
    if ((uintptr_t)d_blob % ENTQ_REGION_ALIGN) return ENTQ_EALIGN;
    for (int j = 0; j < n_jobs; ++j) {
        const entq_pack_adaptive_job &pj = jobs[j];
        const uint32_t C = pj.chunk_symbols;
        if (C == 0 || C % entq::kLanes || C > entq::kMaxChunkSymbols) return ENTQ_EINVAL;
        if (pj.n_symbols == 0) continue;
        if (!pj.d_scratch || !pj.d_n_words || !pj.d_byte_offsets || !pj.d_freq)
            return ENTQ_EINVAL;
        if ((uintptr_t)pj.d_scratch % 16 || (uintptr_t)pj.d_n_words % 4 ||
            (uintptr_t)pj.d_byte_offsets % 8 || (uintptr_t)pj.d_freq % 4)
            return ENTQ_EALIGN;
        if ((pj.n_symbols + C - 1) / C > 0x7FFFFFFFull) return ENTQ_EINVAL;
    }
    entq::PackJobs batch = {};
    uint64_t blocks = 0;
    auto flush = [&]() -> bool {
        if (batch.n_jobs == 0) return true;
        hipLaunchKernelGGL(entq::pack_chunks_batch, dim3((unsigned)blocks), dim3(256), 0,
                           (hipStream_t)stream, batch, static_cast<uint8_t *>(d_blob));
        batch = {};
        blocks = 0;
        return hipGetLastError() == hipSuccess;
    };
    for (int j = 0; j < n_jobs; ++j) {
        const entq_pack_adaptive_job &pj = jobs[j];
        if (pj.n_symbols == 0) continue;
        const uint64_t k = (pj.n_symbols + pj.chunk_symbols - 1) / pj.chunk_symbols;
        if (batch.n_jobs == (uint32_t)entq::kMaxEncJobs || blocks + k > 0x7FFFFFFFull)
            if (!flush()) return ENTQ_EHIP;
        batch.job[batch.n_jobs++] = {static_cast<const uint8_t *>(pj.d_scratch), pj.d_n_words,
                                     pj.d_byte_offsets, pj.d_freq, pj.chunk_symbols,
                                     (uint32_t)blocks};
        blocks += k;
    }
    return flush() ? ENTQ_OK : ENTQ_EHIP;
}

}  // extern "C"

// entq_encode.cpp -- host-side (offline) compression for libentq: symbol
// counts, the 12-bit frequency table and the 64-lane interleaved rANS
// encoder that writes the chunk regions the GPU decoder reads.
//
// The method compresses the flattened 8-bit codes of each weight tensor
// without loss with an ANS coder before the model is deployed [EntQuant,
// "Float8@2bits: Entropy Coding Enables Data-Free Model Compression",
// technical summary §2 "Codificación de Pesos"]; for BF16 weights only the
// exponent byte is coded [DFloat11 write-up, "Formato DFloat11"]. The coder
// is range ANS (Duda 2013) with 64 interleaved states (Giesen 2014); its
// parameters are the library's format, documented in entq.h.
#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "entq.h"
#include "entq_internal.h"

namespace {

int pick_threads(int requested, uint64_t work_items) {
    int n = requested > 0 ? requested : (int)std::thread::hardware_concurrency();
    if (n < 1) n = 1;
    if (n > 64) n = 64;
    if ((uint64_t)n > work_items) n = (int)std::max<uint64_t>(1, work_items);
    return n;
}

template <class F>
void parallel_ranges(int n_threads, uint64_t n, F &&body) {
    if (n_threads <= 1) {
        body(0, (uint64_t)0, n);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(n_threads - 1);
    for (int t = 1; t < n_threads; ++t)
        pool.emplace_back([&, t] { body(t, n * t / n_threads, n * (t + 1) / n_threads); });
    body(0, (uint64_t)0, n / n_threads);
    for (auto &th : pool) th.join();
}

inline uint64_t region_size(uint32_t n_words) {
    uint64_t b = entq::kStateBytes + 2ull * n_words;
    return (b + (ENTQ_REGION_ALIGN - 1)) & ~(uint64_t)(ENTQ_REGION_ALIGN - 1);
}

// Per-symbol coding constants of one table.
struct SymCode {
    uint32_t freq;      // f
    uint32_t start;     // cumulative frequency of the smaller bytes
    uint64_t x_limit;   // states at or above this shed a word first: 2^20 * f
    uint64_t recip;     // floor(2^44 / f) + 1, for exact division (see div_freq)
};

// floor(x / f) for x < 2^32, 1 <= f <= 4096, without a divide instruction:
// x * recip / 2^44 = x / f + e with 0 < e < 2^-12 <= 1/f, and x / f is at
// most (f - 1) / f above its floor, so the floor of the sum is floor(x / f).
inline uint32_t div_freq(uint32_t x, uint64_t recip) {
    return (uint32_t)(((unsigned __int128)x * recip) >> 44);
}

// The coding constants of a table; false if it does not sum to 4096.
bool make_code(const uint16_t freq[256], SymCode code[256]) {
    uint32_t total = 0;
    for (int s = 0; s < 256; ++s) {
        code[s].freq = freq[s];
        code[s].start = total;
        code[s].x_limit = (uint64_t)freq[s] << 20;  // ((L >> 12) << 16) * f
        code[s].recip = freq[s] ? ((1ull << 44) / freq[s]) + 1 : 0;
        total += freq[s];
    }
    return total == entq::kProbScale;
}

// Encodes one chunk: symbols sym[0..n) on lanes i mod 64, walked back to
// front (the decoder reads front to back). Emitted words are stored from the
// end of `scratch` towards its start, so scratch[*first .. cap) ends up in
// decoding order. Returns false if a symbol has frequency 0.
bool encode_chunk(const uint8_t *sym, uint32_t n, const SymCode *code, uint32_t lanes_out[64],
                  uint16_t *scratch, uint32_t cap, uint32_t *first) {
    uint32_t x[64];
    for (int j = 0; j < 64; ++j) x[j] = entq::kStateLow;
    uint32_t w = cap;
    for (uint32_t i = n; i-- > 0;) {
        uint32_t &xs = x[i & 63];
        const SymCode &c = code[sym[i]];
        if (c.freq == 0) return false;
        if ((uint64_t)xs >= c.x_limit) {
            scratch[--w] = (uint16_t)xs;
            xs >>= 16;
        }
        uint32_t q = div_freq(xs, c.recip);
        uint32_t r = xs - q * c.freq;
        xs = (q << entq::kProbBits) + r + c.start;
    }
    std::memcpy(lanes_out, x, sizeof(x));
    *first = w;
    return true;
}

}  // namespace

extern "C" {

entq_status entq_count_symbols(const uint8_t *symbols, uint64_t n, uint64_t counts[256],
                               int n_threads) {
    if (!counts || (n && !symbols)) return ENTQ_EINVAL;
    int nt = pick_threads(n_threads, n / (1u << 20) + 1);
    std::vector<uint64_t> part((size_t)nt * 256, 0);
    parallel_ranges(nt, n, [&](int t, uint64_t b, uint64_t e) {
        uint64_t *h = &part[(size_t)t * 256];
        for (uint64_t i = b; i < e; ++i) h[symbols[i]]++;
    });
    for (int s = 0; s < 256; ++s) {
        uint64_t v = 0;
        for (int t = 0; t < nt; ++t) v += part[(size_t)t * 256 + s];
        counts[s] = v;
    }
    return ENTQ_OK;
}

entq_status entq_build_freq(const uint64_t counts[256], uint16_t freq[256]) {
    if (!counts || !freq) return ENTQ_EINVAL;
    uint64_t total = 0;
    int n_present = 0, only = -1;
    for (int s = 0; s < 256; ++s) {
        total += counts[s];
        if (counts[s]) { n_present++; only = s; }
    }
    std::fill(freq, freq + 256, (uint16_t)0);
    if (n_present == 0) return ENTQ_OK;
    if (n_present == 1) {
        freq[only] = (uint16_t)entq::kProbScale;
        return ENTQ_OK;
    }
    // nearest share of 4096, halves up, at least 1
    int64_t sum = 0;
    for (int s = 0; s < 256; ++s) {
        if (!counts[s]) continue;
        unsigned __int128 num = (unsigned __int128)counts[s] * (2u * entq::kProbScale) + total;
        uint64_t v = (uint64_t)(num / ((unsigned __int128)total * 2u));
        if (v == 0) v = 1;
        freq[s] = (uint16_t)v;
        sum += (int64_t)v;
    }
    // too much: trim the largest frequencies first (smaller byte wins ties)
    while (sum > (int64_t)entq::kProbScale) {
        int arg = -1;
        for (int s = 0; s < 256; ++s)
            if (freq[s] > 1 && (arg < 0 || freq[s] > freq[arg])) arg = s;
        freq[arg]--;
        sum--;
    }
    // too little: the most frequent symbol absorbs the rest
    if (sum < (int64_t)entq::kProbScale) {
        int arg = -1;
        for (int s = 0; s < 256; ++s)
            if (counts[s] && (arg < 0 || counts[s] > counts[arg])) arg = s;
        freq[arg] = (uint16_t)(freq[arg] + (entq::kProbScale - sum));
    }
    return ENTQ_OK;
}

entq_status entq_build_freq_chunks(const uint32_t *counts, uint64_t n_tables, uint16_t *freq,
                                   int n_threads) {
    if (n_tables == 0) return ENTQ_OK;
    if (!counts || !freq) return ENTQ_EINVAL;
    parallel_ranges(pick_threads(n_threads, n_tables / 64 + 1), n_tables,
                    [&](int, uint64_t lo, uint64_t hi) {
                        uint64_t c[256];
                        for (uint64_t t = lo; t < hi; ++t) {
                            for (int s = 0; s < 256; ++s) c[s] = counts[t * 256 + s];
                            entq_build_freq(c, freq + t * 256);
                        }
                    });
    return ENTQ_OK;
}

uint64_t entq_encode_bound(uint64_t n_symbols, uint32_t chunk_symbols) {
    if (chunk_symbols == 0) return 0;
    uint64_t k = (n_symbols + chunk_symbols - 1) / chunk_symbols;
    return k * (entq::kStateBytes + ENTQ_REGION_ALIGN) + 2 * n_symbols;
}


}  // extern "C"

namespace {

// The tensor encoder. freq == nullptr: every chunk is coded with the table of
// its own counts (entq_build_freq), stored as the first ENTQ_TABLE_BYTES of
// its region.
entq_status encode_tensor_impl(const uint8_t *symbols, uint64_t n, uint32_t chunk_symbols,
                               const uint16_t *freq, uint32_t tensor_id,
                               uint64_t base_offset, uint8_t *out, uint64_t out_cap,
                               entq_chunk_desc *chunks_out, uint64_t *bytes_written,
                               int n_threads) {
    if (!bytes_written || (n && (!symbols || !out || !chunks_out)))
        return ENTQ_EINVAL;
    if (chunk_symbols == 0 || chunk_symbols % entq::kLanes || chunk_symbols > entq::kMaxChunkSymbols)
        return ENTQ_EINVAL;
    if (base_offset % ENTQ_REGION_ALIGN) return ENTQ_EALIGN;
    *bytes_written = 0;
    if (n == 0) return ENTQ_OK;
    const bool adaptive = freq == nullptr;
    const uint32_t head = adaptive ? ENTQ_TABLE_BYTES : 0;
    SymCode shared[256];
    if (!adaptive && !make_code(freq, shared)) return ENTQ_EBADTABLE;

    const uint64_t n_chunks = (n + chunk_symbols - 1) / chunk_symbols;
    const int nt = pick_threads(n_threads, n_chunks);
    struct Part {
        std::vector<uint8_t> bytes;
        bool ok = true;
    };
    std::vector<Part> parts(nt);
    std::vector<uint64_t> local_off(n_chunks);
    parallel_ranges(nt, n_chunks, [&](int t, uint64_t kb, uint64_t ke) {
        Part &part = parts[t];
        // worst case (one word per symbol); untouched pages cost nothing
        part.bytes.reserve((ke - kb) * (head + entq::kStateBytes + ENTQ_REGION_ALIGN + 2ull * chunk_symbols));
        std::vector<uint16_t> scratch(chunk_symbols);
        uint32_t lanes[64];
        SymCode own[256];
        uint16_t own_freq[256];
        for (uint64_t k = kb; k < ke && part.ok; ++k) {
            const uint64_t e0 = k * chunk_symbols;
            const uint32_t cn = (uint32_t)std::min<uint64_t>(chunk_symbols, n - e0);
            const SymCode *code = shared;
            if (adaptive) {
                uint64_t counts[256] = {0};
                for (uint32_t i = 0; i < cn; ++i) counts[symbols[e0 + i]]++;
                entq_build_freq(counts, own_freq);
                make_code(own_freq, own);
                code = own;
            }
            uint32_t first = 0;
            if (!encode_chunk(symbols + e0, cn, code, lanes, scratch.data(), chunk_symbols, &first)) {
                part.ok = false;
                break;
            }
            const uint32_t nw = chunk_symbols - first;
            const uint64_t at = part.bytes.size();
            part.bytes.resize(at + head + region_size(nw), 0);
            uint8_t *r = part.bytes.data() + at;
            if (adaptive) std::memcpy(r, own_freq, ENTQ_TABLE_BYTES);  // little-endian host
            std::memcpy(r + head, lanes, entq::kStateBytes);
            std::memcpy(r + head + entq::kStateBytes, scratch.data() + first, 2ull * nw);
            local_off[k] = at;
            entq_chunk_desc &d = chunks_out[k];
            d.tensor = tensor_id;
            d.n_symbols = cn;
            d.n_words = nw;
            d.reserved = 0;
            d.elem_offset = e0;
        }
    });
    uint64_t total_bytes = 0;
    for (auto &p : parts) {
        if (!p.ok) return ENTQ_ESYMBOL;
        total_bytes += p.bytes.size();
    }
    if (total_bytes > out_cap) return ENTQ_EINVAL;
    // place each thread's run of regions after the previous ones
    std::vector<uint64_t> part_base(nt, 0);
    for (int t = 1; t < nt; ++t) part_base[t] = part_base[t - 1] + parts[t - 1].bytes.size();
    parallel_ranges(nt, (uint64_t)nt, [&](int, uint64_t tb, uint64_t te) {
        for (uint64_t t = tb; t < te; ++t)
            if (!parts[t].bytes.empty())
                std::memcpy(out + part_base[t], parts[t].bytes.data(), parts[t].bytes.size());
    });
    for (int t = 0; t < nt; ++t) {
        uint64_t kb = n_chunks * t / nt, ke = n_chunks * (t + 1) / nt;
        for (uint64_t k = kb; k < ke; ++k)
            chunks_out[k].byte_offset = base_offset + part_base[t] + local_off[k];
    }
    *bytes_written = total_bytes;
    return ENTQ_OK;
}

}  // namespace

extern "C" {

entq_status entq_encode_tensor(const uint8_t *symbols, uint64_t n, uint32_t chunk_symbols,
                               const uint16_t freq[256], uint32_t tensor_id,
                               uint64_t base_offset, uint8_t *out, uint64_t out_cap,
                               entq_chunk_desc *chunks_out, uint64_t *bytes_written,
                               int n_threads) {
    if (!freq) return ENTQ_EINVAL;
    return encode_tensor_impl(symbols, n, chunk_symbols, freq, tensor_id, base_offset, out,
                              out_cap, chunks_out, bytes_written, n_threads);
}

entq_status entq_encode_tensor_adaptive(const uint8_t *symbols, uint64_t n,
                                        uint32_t chunk_symbols, uint32_t tensor_id,
                                        uint64_t base_offset, uint8_t *out, uint64_t out_cap,
                                        entq_chunk_desc *chunks_out, uint64_t *bytes_written,
                                        int n_threads) {
    return encode_tensor_impl(symbols, n, chunk_symbols, nullptr, tensor_id, base_offset, out,
                              out_cap, chunks_out, bytes_written, n_threads);
}

uint64_t entq_encode_bound_adaptive(uint64_t n_symbols, uint32_t chunk_symbols) {
    if (chunk_symbols == 0) return 0;
    uint64_t k = (n_symbols + chunk_symbols - 1) / chunk_symbols;
    return entq_encode_bound(n_symbols, chunk_symbols) + k * ENTQ_TABLE_BYTES;
}

entq_status entq_bf16_split(const uint16_t *w, uint64_t n, uint8_t *exp_out, uint8_t *sm_out,
                            int n_threads) {
    if (n && (!w || !exp_out || !sm_out)) return ENTQ_EINVAL;
    int nt = pick_threads(n_threads, n / (1u << 20) + 1);
    parallel_ranges(nt, n, [&](int, uint64_t b, uint64_t e) {
        for (uint64_t i = b; i < e; ++i) {
            const uint16_t v = w[i];
            exp_out[i] = (uint8_t)(v >> 7);
            sm_out[i] = (uint8_t)(((v >> 8) & 0x80) | (v & 0x7F));
        }
    });
    return ENTQ_OK;
}

// Tile order of one tensor (see include/entq.h): chunk k = (band b, column
// chunk c), inside it position 256 t + 64 s + l holds row 16 b + l % 16,
// column c C + 16 t + 4 (l / 16) + s.
entq_status entq_tile_order(const uint8_t *codes, uint32_t rows, uint32_t cols,
                            uint32_t chunk_cols, uint8_t *out, int n_threads) {
    if (rows % 16 || chunk_cols == 0 || chunk_cols % 16 || cols % chunk_cols) return ENTQ_EINVAL;
    const uint64_t n = (uint64_t)rows * cols;
    if (n && (!codes || !out)) return ENTQ_EINVAL;
    const uint32_t ncc = cols / chunk_cols;
    const uint64_t chunks = (uint64_t)(rows / 16) * ncc;
    const uint64_t per = 16ull * chunk_cols;
    int nt = pick_threads(n_threads, n / (1u << 20) + 1);
    parallel_ranges(nt, chunks, [&](int, uint64_t kb, uint64_t ke) {
        for (uint64_t k = kb; k < ke; ++k) {
            const uint64_t b = k / ncc, c = k % ncc;
            uint8_t *dst = out + k * per;
            for (uint64_t p = 0; p < per; ++p) {
                const uint64_t t = p >> 8, sidx = (p >> 6) & 3, l = p & 63;
                const uint64_t row = 16 * b + (l & 15);
                const uint64_t col = c * chunk_cols + 16 * t + 4 * (l >> 4) + sidx;
                dst[p] = codes[row * cols + col];
            }
        }
    });
    return ENTQ_OK;
}

}  // extern "C"

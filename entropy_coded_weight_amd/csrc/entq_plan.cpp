// entq_plan.cpp -- validation of a batch of coded tensors and construction of
// the decoder's device-side tables, chunk list and workgroup tasks.
//
// A batch is what one decode launch covers: typically all weight matrices of
// one transformer block, decoded together just before the block runs
// [DFloat11 write-up, "Descompresión por bloque transformer"; EntQuant,
// "Float8@2bits ...", technical summary §2 "Decodificación en Tiempo de
// Inferencia"]. Each chunk decodes independently of the others, which is
// what lets the batch spread over the whole GPU [EntroLLM summary,
// "Metodología" item 3].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "entq.h"
#include "entq_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct Layout {
    size_t tables, tensors, chunks, tasks, total;
};

Layout layout_for(int n_tensors, int64_t n_chunks, int64_t n_tasks) {
    Layout l;
    l.tables = 0;
    l.tensors = l.tables + align_up((size_t)n_tensors * entq::kProbScale * sizeof(entq::SlotEntry));
    l.chunks = l.tensors + align_up((size_t)n_tensors * sizeof(entq::DevTensor));
    l.tasks = l.chunks + align_up((size_t)n_chunks * sizeof(entq::DevChunk));
    l.total = l.tasks + align_up((size_t)n_tasks * sizeof(entq::DevTask));
    if (l.total == 0) l.total = kAlign;
    return l;
}

uint64_t region_size(uint32_t n_words) {
    uint64_t b = entq::kStateBytes + 2ull * n_words;
    return (b + (ENTQ_REGION_ALIGN - 1)) & ~(uint64_t)(ENTQ_REGION_ALIGN - 1);
}

}  // namespace

extern "C" {

size_t entq_plan_workspace_bytes(int n_tensors, int64_t n_chunks) {
    if (n_tensors < 0 || n_chunks < 0) return 0;
    // at most one task per chunk
    return layout_for(n_tensors, n_chunks, n_chunks).total;
}

const char *entq_status_str(entq_status s) {
    switch (s) {
    case ENTQ_OK: return "ok";
    case ENTQ_EINVAL: return "invalid argument";
    case ENTQ_EBADTABLE: return "frequency table does not sum to 4096";
    case ENTQ_EBADINDEX: return "chunk index does not tile the tensors";
    case ENTQ_EALIGN: return "misaligned region or buffer";
    case ENTQ_EWORKSPACE: return "workspace too small";
    case ENTQ_EHIP: return "HIP call failed";
    case ENTQ_ENOMEM: return "out of host memory";
    case ENTQ_ESYMBOL: return "a coded symbol has frequency 0";
    case ENTQ_ETOOLARGE: return "request exceeds the library's static scratch";
    }
    return "unknown status";
}

}  // extern "C"

namespace {

// The plan builder behind entq_plan and entq_plan_adaptive. adaptive: every
// chunk region starts with its own table (freq_tables unused), the decode
// goes through decode_adaptive, which needs whole 256-symbol blocks.
entq_status plan_impl(const entq_tensor_desc *tensors, int n_tensors, const uint16_t *freq_tables,
                      const entq_chunk_desc *chunk_index, int64_t n_chunks, uint64_t blob_bytes,
                      void *d_workspace, size_t workspace_bytes, void *stream, entq_plan_t **out,
                      bool adaptive) {
    if (!out) return ENTQ_EINVAL;
    *out = nullptr;
    if (n_tensors < 0 || n_chunks < 0) return ENTQ_EINVAL;
    if (n_tensors > 0 && (!tensors || (!adaptive && !freq_tables))) return ENTQ_EINVAL;
    if (n_chunks > 0 && !chunk_index) return ENTQ_EINVAL;
    if (n_chunks > (int64_t)UINT32_MAX) return ENTQ_EINVAL;
    if (!d_workspace) return ENTQ_EINVAL;
    if ((uintptr_t)d_workspace % kAlign) return ENTQ_EALIGN;

    // ---- tensors
    uint64_t out_elems = 0, scale_rows = 0;
    uint32_t kinds_mask = 0;
    int n_tiled = 0, n_nonempty = 0;
    for (int t = 0; t < n_tensors; ++t) {
        const entq_tensor_desc &td = tensors[t];
        if (td.kind & ~(0xFFu | ENTQ_LAYOUT_TILES)) return ENTQ_EINVAL;
        const uint32_t kind = td.kind & 0xFFu;
        if (kind > ENTQ_SYM_BF16EXP) return ENTQ_EINVAL;
        if (td.kind & ENTQ_LAYOUT_TILES) {
            // 16-row bands of chunk_symbols / 16 columns, whole 16 x 16 tiles
            if (adaptive) return ENTQ_EINVAL;
            if (td.rows % 16 || td.chunk_symbols % entq::kBlockSyms) return ENTQ_EINVAL;
            if (td.cols % (td.chunk_symbols / 16)) return ENTQ_EINVAL;
            if (td.out_elem_offset % 16) return ENTQ_EINVAL;  // 16-byte output rows
        }
        if (td.chunk_symbols == 0 || td.chunk_symbols % entq::kLanes ||
            td.chunk_symbols > entq::kMaxChunkSymbols)
            return ENTQ_EINVAL;
        if ((uint64_t)td.rows * td.cols != td.n_symbols) return ENTQ_EINVAL;
        if (td.n_symbols == 0) continue;
        if (adaptive) {
            // whole 256-symbol blocks; bf16 rows (scales) of whole blocks
            if (td.chunk_symbols % entq::kBlockSyms || td.out_elem_offset % 16) return ENTQ_EINVAL;
            if (kind != ENTQ_SYM_BF16EXP && td.cols % entq::kBlockSyms) return ENTQ_EINVAL;
        } else {
            uint32_t sum = 0;
            for (int s = 0; s < 256; ++s) sum += freq_tables[(size_t)t * 256 + s];
            if (sum != entq::kProbScale) return ENTQ_EBADTABLE;
        }
        kinds_mask |= 1u << kind;
        if (td.kind & ENTQ_LAYOUT_TILES) kinds_mask |= entq::kTilesBit;
        n_tiled += (td.kind & ENTQ_LAYOUT_TILES) ? 1 : 0;
        ++n_nonempty;
        if (td.out_elem_offset > UINT64_MAX - td.n_symbols) return ENTQ_EINVAL;
        out_elems = std::max(out_elems, td.out_elem_offset + td.n_symbols);
        scale_rows = std::max(scale_rows, td.scale_row_offset + td.rows);
    }
    // outputs of different tensors must not overlap
    {
        std::vector<std::pair<uint64_t, uint64_t>> spans;
        for (int t = 0; t < n_tensors; ++t)
            if (tensors[t].n_symbols)
                spans.emplace_back(tensors[t].out_elem_offset, tensors[t].n_symbols);
        std::sort(spans.begin(), spans.end());
        for (size_t i = 1; i < spans.size(); ++i)
            if (spans[i - 1].first + spans[i - 1].second > spans[i].first) return ENTQ_EINVAL;
    }

    // ---- chunks: each tensor's chunks tile [0, n_symbols) exactly
    std::vector<std::vector<int64_t>> slot_of(n_tensors);
    for (int t = 0; t < n_tensors; ++t) {
        const uint64_t k = (tensors[t].n_symbols + tensors[t].chunk_symbols - 1) / tensors[t].chunk_symbols;
        if (k > (uint64_t)n_chunks) return ENTQ_EBADINDEX;
        slot_of[t].assign(k, -1);
    }
    for (int64_t c = 0; c < n_chunks; ++c) {
        const entq_chunk_desc &cd = chunk_index[c];
        if (cd.tensor >= (uint32_t)n_tensors) return ENTQ_EBADINDEX;
        const entq_tensor_desc &td = tensors[cd.tensor];
        if (cd.byte_offset % ENTQ_REGION_ALIGN) return ENTQ_EALIGN;
        if (cd.n_symbols == 0 || cd.n_symbols > td.chunk_symbols) return ENTQ_EBADINDEX;
        if (cd.n_words > cd.n_symbols) return ENTQ_EBADINDEX;
        if (cd.elem_offset % td.chunk_symbols || cd.elem_offset >= td.n_symbols) return ENTQ_EBADINDEX;
        const uint64_t expect = std::min<uint64_t>(td.chunk_symbols, td.n_symbols - cd.elem_offset);
        if (cd.n_symbols != expect) return ENTQ_EBADINDEX;
        const uint64_t rb = region_size(cd.n_words) + (adaptive ? ENTQ_TABLE_BYTES : 0);
        if (cd.byte_offset > blob_bytes || rb > blob_bytes - cd.byte_offset)
            return ENTQ_EBADINDEX;
        int64_t &slot = slot_of[cd.tensor][cd.elem_offset / td.chunk_symbols];
        if (slot >= 0) return ENTQ_EBADINDEX;  // two chunks for one place
        slot = c;
    }
    for (int t = 0; t < n_tensors; ++t)
        for (int64_t s : slot_of[t])
            if (s < 0) return ENTQ_EBADINDEX;  // a hole

    // ---- task groups: block- and row-aligned tensors first, then
    // block-aligned, then the rest (the launcher picks a kernel per group)
    auto group_of = [&](int t) {
        const entq_tensor_desc &td = tensors[t];
        // the streaming kernel writes 4 outputs and reads 4 sign+mantissa
        // bytes per lane and block (vector accesses): chunk sizes must be
        // whole blocks and outputs 16-aligned
        if (td.chunk_symbols % entq::kBlockSyms || td.out_elem_offset % 16) return 2;
        return (td.cols % entq::kBlockSyms) ? 1 : 0;
    };
    std::vector<int> order;
    for (int g = 0; g < 3; ++g)
        for (int t = 0; t < n_tensors; ++t)
            if (group_of(t) == g && !slot_of[t].empty()) order.push_back(t);
    std::vector<int64_t> chunk_base(n_tensors, 0);  // first DevChunk of each tensor
    {
        int64_t c = 0;
        for (int t : order) { chunk_base[t] = c; c += (int64_t)slot_of[t].size(); }
    }
    // Tasks. A chunk costs about its symbol count, so a launch finishes when
    // its busiest workgroup does: when a group holds more chunks than there
    // are resident workgroups, every resident workgroup gets one task, the
    // tensors sharing the workgroups in proportion to their symbols and each
    // splitting its (equal) chunks into near-equal runs; otherwise every
    // chunk is a task of its own (latency-bound, so spread over as many CUs
    // as possible). (Sharing by chunk count instead made a 70B-shaped layer
    // in one-row chunks take 774 instead of 469 us: the down projection's
    // chunks are 3.5 times longer than the others'.)
    const int64_t slots = std::max<int64_t>(1, entq::resident_workgroups());
    std::vector<entq::DevTask> task_list;
    int64_t group_end[3] = {0, 0, 0};
    for (int g = 0; g < 3; ++g) {
        std::vector<int> tens;
        int64_t K = 0;
        for (int t : order)
            if (group_of(t) == g) { tens.push_back(t); K += (int64_t)slot_of[t].size(); }
        std::vector<int64_t> share(tens.size());
        if (K <= slots) {
            for (size_t i = 0; i < tens.size(); ++i) share[i] = (int64_t)slot_of[tens[i]].size();
        } else {
            // largest-remainder apportionment of the slots, at least one each
            std::vector<std::pair<double, size_t>> frac;
            int64_t given = 0;
            double S = 0;
            for (int t : tens) S += (double)tensors[t].n_symbols;
            for (size_t i = 0; i < tens.size(); ++i) {
                const double q = (double)slots * (double)tensors[tens[i]].n_symbols / S;
                share[i] = std::max<int64_t>(1, (int64_t)q);
                given += share[i];
                frac.emplace_back(q - (double)(int64_t)q, i);
            }
            std::sort(frac.begin(), frac.end(), [](auto &a, auto &b) { return a.first > b.first; });
            for (size_t j = 0; given < slots && j < frac.size(); ++j, ++given) share[frac[j].second]++;
        }
        for (size_t i = 0; i < tens.size(); ++i) {
            const int t = tens[i];
            const int64_t k = (int64_t)slot_of[t].size();
            const int64_t parts = std::min(share[i], k);
            for (int64_t j = 0; j < parts; ++j) {
                const int64_t lo = k * j / parts, hi = k * (j + 1) / parts;
                entq::DevTask d;
                d.first_chunk = (uint32_t)(chunk_base[t] + lo);
                d.n_chunks = (uint32_t)(hi - lo);
                d.tensor = (uint32_t)t;
                d.pad = 0;
                task_list.push_back(d);
            }
        }
        group_end[g] = (int64_t)task_list.size();
    }
    const int64_t n_tasks = (int64_t)task_list.size();

    const Layout lay = layout_for(n_tensors, n_chunks, n_tasks);
    if (workspace_bytes < lay.total) return ENTQ_EWORKSPACE;

    // ---- host image of the workspace
    uint8_t *img = (uint8_t *)std::calloc(1, lay.total);
    if (!img) return ENTQ_ENOMEM;
    auto *tables = reinterpret_cast<entq::SlotEntry *>(img + lay.tables);
    auto *dten = reinterpret_cast<entq::DevTensor *>(img + lay.tensors);
    auto *dch = reinterpret_cast<entq::DevChunk *>(img + lay.chunks);
    auto *dtask = reinterpret_cast<entq::DevTask *>(img + lay.tasks);
    for (int t = 0; t < n_tensors; ++t) {
        const uint16_t *f = freq_tables + (size_t)t * 256;
        entq::SlotEntry *T = tables + (size_t)t * entq::kProbScale;
        if (tensors[t].n_symbols && !adaptive) {
            uint32_t start = 0;
            for (uint32_t s = 0; s < 256; ++s) {
                for (uint32_t k = 0; k < f[s]; ++k) {
                    T[start + k].lo = (uint32_t)f[s] | (s << 24);
                    T[start + k].hi = k;  // slot - cum[s]
                }
                start += f[s];
            }
        }
        dten[t].cols = tensors[t].cols;
        dten[t].kind = tensors[t].kind & 0xFFu;
    }
    for (int t : order) {
        const entq_tensor_desc &td = tensors[t];
        int64_t c = chunk_base[t];
        for (int64_t s : slot_of[t]) {
            const entq_chunk_desc &cd = chunk_index[s];
            entq::DevChunk &d = dch[c++];
            d.byte_offset = cd.byte_offset;
            d.out_elem = td.out_elem_offset + cd.elem_offset;
            d.scale_row = td.scale_row_offset + (td.cols ? cd.elem_offset / td.cols : 0);
            d.col0 = td.cols ? (uint32_t)(cd.elem_offset % td.cols) : 0;
            d.n_symbols = cd.n_symbols;
            d.n_words = cd.n_words;
            d.status_index = (uint32_t)s;
            d.tensor = (uint32_t)t;
        }
    }
    std::copy(task_list.begin(), task_list.end(), dtask);

    std::vector<entq::HostTensor> host_tensors;
    try {
        host_tensors.resize(n_tensors);
    } catch (...) {
        std::free(img);
        return ENTQ_ENOMEM;
    }
    for (int t = 0; t < n_tensors; ++t) {
        const entq_tensor_desc &td = tensors[t];
        host_tensors[t] = {td.kind & 0xFFu, td.rows, td.cols, td.chunk_symbols, td.n_symbols,
                           chunk_base[t], (int64_t)slot_of[t].size(), td.out_elem_offset,
                           td.scale_row_offset, (td.kind & ENTQ_LAYOUT_TILES) != 0};
    }
    // the plan object exists before the copy is enqueued, so that no failure
    // after it has to free the copy's source
    entq_plan_t *p = new (std::nothrow) entq_plan_t;
    if (!p) {
        std::free(img);
        return ENTQ_ENOMEM;
    }
    // the host image stays alive until the copy from it has completed: destroy
    // waits for this event before freeing it
    hipEvent_t ev = nullptr;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
        delete p;
        std::free(img);
        return ENTQ_EHIP;
    }
    if (hipMemcpyAsync(d_workspace, img, lay.total, hipMemcpyHostToDevice, (hipStream_t)stream) !=
            hipSuccess ||
        hipEventRecord(ev, (hipStream_t)stream) != hipSuccess) {
        // cleanup after a failure: errors here change nothing the caller can act on
        (void)hipStreamSynchronize((hipStream_t)stream);  // a copy may have been enqueued
        (void)hipEventDestroy(ev);
        delete p;
        std::free(img);
        return ENTQ_EHIP;
    }
    p->upload_done = ev;
    uint8_t *ws = (uint8_t *)d_workspace;
    p->n_tensors = n_tensors;
    p->n_chunks = n_chunks;
    p->n_tasks = n_tasks;
    p->n_tasks_rows = group_end[0];
    p->n_tasks_blocks = group_end[1];
    p->max_task_chunks_rows = p->max_task_chunks_blocks = 0;
    for (int64_t k = 0; k < group_end[1]; ++k) {
        const uint32_t c = task_list[k].n_chunks;
        if (k < group_end[0]) p->max_task_chunks_rows = std::max(p->max_task_chunks_rows, c);
        p->max_task_chunks_blocks = std::max(p->max_task_chunks_blocks, c);
    }
    p->blob_bytes = blob_bytes;
    p->out_elems = out_elems;
    p->scale_rows = scale_rows;
    p->kinds_mask = kinds_mask;
    p->mixed_layouts = n_tiled > 0 && n_tiled < n_nonempty;
    p->d_tables = reinterpret_cast<const entq::SlotEntry *>(ws + lay.tables);
    p->d_tensors = reinterpret_cast<const entq::DevTensor *>(ws + lay.tensors);
    p->d_chunks = reinterpret_cast<const entq::DevChunk *>(ws + lay.chunks);
    p->d_tasks = reinterpret_cast<const entq::DevTask *>(ws + lay.tasks);
    p->host_staging = img;
    p->host_tensors = std::move(host_tensors);
    p->adaptive = adaptive;
    *out = p;
    return ENTQ_OK;
}

}  // namespace

extern "C" {

entq_status entq_plan(const entq_tensor_desc *tensors, int n_tensors, const uint16_t *freq_tables,
                      const entq_chunk_desc *chunk_index, int64_t n_chunks, uint64_t blob_bytes,
                      void *d_workspace, size_t workspace_bytes, void *stream, entq_plan_t **out) {
    return plan_impl(tensors, n_tensors, freq_tables, chunk_index, n_chunks, blob_bytes,
                     d_workspace, workspace_bytes, stream, out, false);
}

entq_status entq_plan_adaptive(const entq_tensor_desc *tensors, int n_tensors,
                               const entq_chunk_desc *chunk_index, int64_t n_chunks,
                               uint64_t blob_bytes, void *d_workspace, size_t workspace_bytes,
                               void *stream, entq_plan_t **out) {
    return plan_impl(tensors, n_tensors, nullptr, chunk_index, n_chunks, blob_bytes, d_workspace,
                     workspace_bytes, stream, out, true);
}

void entq_plan_destroy(entq_plan_t *plan) {
    if (!plan) return;
    if (plan->upload_done) {
        // destroy cannot report errors; waiting is what keeps host_staging valid
        (void)hipEventSynchronize((hipEvent_t)plan->upload_done);  // the upload read host_staging
        (void)hipEventDestroy((hipEvent_t)plan->upload_done);
    }
    std::free(plan->host_staging);
    delete plan;
}

entq_status entq_plan_info(const entq_plan_t *plan, uint64_t *out_elems, uint64_t *scale_rows,
                           int64_t *n_chunks, int *n_tensors, uint64_t *blob_bytes) {
    if (!plan) return ENTQ_EINVAL;
    if (out_elems) *out_elems = plan->out_elems;
    if (scale_rows) *scale_rows = plan->scale_rows;
    if (n_chunks) *n_chunks = plan->n_chunks;
    if (n_tensors) *n_tensors = plan->n_tensors;
    if (blob_bytes) *blob_bytes = plan->blob_bytes;
    return ENTQ_OK;
}

entq_status entq_decode(const entq_plan_t *plan, const void *d_compressed, void *d_out,
                        entq_outkind out_kind, const float *d_scales, int32_t *d_chunk_status,
                        void *stream) {
    if (!plan) return ENTQ_EINVAL;
    if (out_kind != ENTQ_OUT_CODES && out_kind != ENTQ_OUT_BF16) return ENTQ_EINVAL;
    if (plan->n_chunks == 0) return ENTQ_OK;
    if (!d_compressed || !d_out) return ENTQ_EINVAL;
    if ((uintptr_t)d_compressed % ENTQ_REGION_ALIGN || (uintptr_t)d_out % 16) return ENTQ_EALIGN;
    int mode = entq::kModeCodes;
    if (out_kind == ENTQ_OUT_BF16) {
        if (plan->kinds_mask & (1u << ENTQ_SYM_BF16EXP)) return ENTQ_EINVAL;
        if (!d_scales) return ENTQ_EINVAL;
        if ((uintptr_t)d_scales % 4) return ENTQ_EALIGN;
        mode = entq::kModeBf16;
    }
    if (plan->kinds_mask & entq::kTilesBit) {  // row-major outputs of tile-ordered tensors
        if (plan->mixed_layouts) return ENTQ_EINVAL;
        return (entq_status)entq::launch_tile_decode(plan, mode, d_compressed, d_out, d_scales,
                                                     nullptr, d_chunk_status, stream);
    }
    if (plan->adaptive)
        return (entq_status)entq::launch_decode_adaptive(plan, mode, d_compressed, d_out,
                                                         d_scales, nullptr, d_chunk_status,
                                                         stream);
    return (entq_status)entq::launch_decode(plan, mode, d_compressed, d_out, d_scales, nullptr,
                                            d_chunk_status, stream);
}

entq_status entq_decode_bf16_split(const entq_plan_t *plan, const void *d_exp_stream,
                                   const uint8_t *d_signmant, uint16_t *d_out,
                                   int32_t *d_chunk_status, void *stream) {
    if (!plan) return ENTQ_EINVAL;
    if (plan->kinds_mask & ~((1u << ENTQ_SYM_BF16EXP) | entq::kTilesBit)) return ENTQ_EINVAL;
    if (plan->n_chunks == 0) return ENTQ_OK;
    if (!d_exp_stream || !d_signmant || !d_out) return ENTQ_EINVAL;
    if ((uintptr_t)d_exp_stream % ENTQ_REGION_ALIGN || (uintptr_t)d_out % 16 ||
        (uintptr_t)d_signmant % 16)
        return ENTQ_EALIGN;
    if (plan->kinds_mask & entq::kTilesBit) {  // row-major outputs of tile-ordered tensors
        if (plan->mixed_layouts) return ENTQ_EINVAL;
        return (entq_status)entq::launch_tile_decode(plan, entq::kModeSplit, d_exp_stream, d_out,
                                                     nullptr, d_signmant, d_chunk_status,
                                                     stream);
    }
    if (plan->adaptive)
        return (entq_status)entq::launch_decode_adaptive(plan, entq::kModeSplit, d_exp_stream,
                                                         d_out, nullptr, d_signmant,
                                                         d_chunk_status, stream);
    return (entq_status)entq::launch_decode(plan, entq::kModeSplit, d_exp_stream, d_out, nullptr,
                                            d_signmant, d_chunk_status, stream);
}

}  // extern "C"

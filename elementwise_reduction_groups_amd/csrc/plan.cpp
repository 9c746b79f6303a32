// Launch planning: which kernel shape a validated group gets (pointwise,
// register rows, tiled rows, tree-mapped) and its launch layout (vector
// width, lanes a row, workgroup size, tiles and caches, persistent rows,
// XCD mapping), from the shapes alone unless PSK_LAYOUT overrides a choice.
// Every choice here changes no element that is computed; the ones that
// change a reduction's bracketing are listed with the override keys below.
//
// Host-only: nothing here calls HIP.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "psk_internal.h"

namespace psk {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Layout overrides for measurement, "key=value" pairs separated by commas in
// PSK_LAYOUT (an unknown or out-of-range value falls back to the default):
//   every kernel: nt=0|1 (nontemporal accesses), bnt=0|1 (nontemporal loads
//     also for broadcast inputs, which other rows read again), fexp=0|1
//     (the split-product exponential for a softmax's f32 exp, else the
//     library's), ftanh=0|1|2 (tanh: the library's, the emitted one, the
//     emitted one without its wave-uniform branch), xcd=0|1 (XCD-contiguous block mapping), block=64..1024
//     (threads per workgroup);
//   tree kernels: tper=2|4|8|16 (elements per thread);
//   stores: sc1=0|1 (relaxed stores of device scope instead of nontemporal
//     ones; 16 bytes go as two of 8), vbytes=8 (8-byte vectors where no
//     byte mask is read);
//   the AdamW kernel: axcd=0|1 (XCD-contiguous block mapping);
//   row kernels: epl (elements of output a lane aims for), lanes=16|32|
//     64..1024, epmax (most elements a lane holds before the tiled kernel
//     takes over, default 32), persist=k (k persistent workgroups a CU),
//     pf=1..4 (rows a persistent workgroup loads ahead), tiled=1 (force the
//     tiled kernel), split=0 (no split rows), sept (elements a lane of a
//     split row holds), slanes=256|512|1024 (lanes of a split row's
//     workgroup), xmap=0|1 (a split row's workgroups on one XCD;
//     measured at [8192,131072] f32: 1.461 / 1.457 ms exact, 1.507 / 1.553
//     ms online with / without);
//   tiled kernel: lanes=64..1024, tn (vectors a lane per tile), tcache=0|1
//     (cached loads before the last phase), rc / lc (tiles kept in
//     registers / LDS), wpe / wmin (most / fewest waves a SIMD), alt=0|1
//     (odd phases walk the tiles last to first), mu / lu (unroll of the
//     loops over tiles read from memory / kept in LDS).
// A layout never changes which elements are computed; lanes, epl, epmax,
// tiled, tn and alt change a reduction's bracketing (within tolerance), fexp
// an exponential's last bits and ftanh=0 a tanh's (within tolerance), the
// others change no bit.
int layout_value(const char* key, int dflt)
{
    const char* env = std::getenv("PSK_LAYOUT");
    if (!env) return dflt;
    std::string s(env), k = std::string(key) + "=";
    size_t pos = 0;
    while (pos < s.size()) {
        size_t end = s.find(',', pos);
        if (end == std::string::npos) end = s.size();
        std::string item = s.substr(pos, end - pos);
        if (item.compare(0, k.size(), k) == 0) return std::atoi(item.c_str() + k.size());
        pos = end + 1;
    }
    return dflt;
}

std::string KernelPlan::key() const
{
    char b[200];
    std::snprintf(b, sizeof b, "k%d v%d b%d l%d n%d nt%d sc%d x%d g%lld t%d c%d w%d m%d p%d r%d s%d bn%d fe%d ft%d",
                  kind, vec, block, lanes, nv, (int)nt, (int)sc1, (int)xcd, (long long)blocks, tiles, (int)tcache,
                  wpe, wmin, persist, rcache, lcache, (int)bnt, (int)fexp, ftanh);
    if (kind == 4) return std::string(b) + " K" + std::to_string(split);
    if (persist) return std::string(b) + " pf" + std::to_string(pf);
    return kind == 3 ? std::string(b) + (alt ? " a1" : " a0") + " u" + std::to_string(munroll) + " y" +
                           std::to_string(lunroll)
                     : std::string(b);
}

KernelPlan plan_kernel(const Analysis& an, bool allow_vector, int split_ept)
{
    KernelPlan p;
    int V = an.out_dtype == PSK_BF16 ? 8 : 4;
    {
        // vbytes=8 (measurement): 8-byte vectors, where no byte mask is read
        // (a mask's vector would be narrower than its 4-byte load)
        bool u8 = false;
        for (const InputInfo& in : an.inputs) u8 = u8 || (in.used && in.dtype == PSK_U8);
        if (layout_value("vbytes", 16) == 8 && !u8 && !an.tree) V /= 2;
    }
    // 16-byte accesses where every per-element input allows them: a
    // last-axis step of 1 and row starts at whole vectors
    p.vec = (allow_vector && an.cols % V == 0 && inputs_vector_ok(an, V)) ? V : 1;
    p.nt = layout_value("nt", 1) != 0;
    p.sc1 = layout_value("sc1", 0) != 0;   // trees choose their own below
    p.bnt = layout_value("bnt", 0) != 0;
    p.fexp = layout_value("fexp", 1) != 0;
    p.ftanh = layout_value("ftanh", 1);
    if (p.ftanh < 0 || p.ftanh > 2) p.ftanh = 1;
    if (an.tree) {
        // Each thread takes `vec` consecutive elements, the fewest of 2, 4,
        // 8, 16 that move at least 40 bytes.  Measured on the 887M-element
        // Llama tree: an SGD step (6 bytes per element) runs at 4.6 / 6.4 /
        // 5.3 TB/s with 4 / 8 / 16, AdamW (22 bytes) at 6.14 / 5.99 TB/s with
        // 2 / 4.  A chunk splits into whole workgroups, which reach the XCDs
        // in the dispatcher's round-robin order: with 64-thread workgroups
        // SGD runs at 6.58 TB/s and AdamW at 6.45, against 6.24 / 6.46 with
        // 128 threads, 6.37 / 6.26 with 256, and 6.47 / 6.09 (128 threads)
        // when each XCD takes a contiguous eighth of the chunks.
        p.kind = 2;
        auto size_of = [](psk_dtype d) { return d == PSK_BF16 ? 2 : 4; };
        int bytes = size_of(an.out_dtype);
        for (const InputInfo& in : an.inputs)
            if (in.used && in.kind != InKind::Scalar) bytes += size_of(in.dtype);
        for (const auto& x : an.extras) bytes += size_of(x.dtype);
        int per = 2;
        while (per < 16 && per * bytes < 40) per *= 2;
        per = layout_value("tper", per);
        if (per != 2 && per != 4 && per != 8 && per != 16) per = 4;
        int block = layout_value("block", 64);
        if (block < 64 || block > 256 || (block & (block - 1))) block = 64;
        p.vec = per;
        p.block = block;
        p.blocks = PSK_TREE_CHUNK / (block * per);   // workgroups per chunk
        p.xcd = layout_value("xcd", 0) != 0;
        // Stores of device scope (the sc1 cache policy) where every output
        // moves at most 8 bytes a thread, so that one store instruction
        // covers whole lines: AdamW as a group (bf16 theta', f32 m', v', 2
        // elements a thread) 3.06 -> 2.96 ms after the per-group flush and
        // 3.29 -> 3.00 ms back to back, as for the hand-written kernel; a
        // 16-byte store split in two 8-byte ones halves SGD's rate, and SGD
        // at 4 elements a thread (8-byte stores) runs at 5.84 TB/s with
        // them against 6.47 at 8 (16-byte nontemporal stores)
        int widest = size_of(an.out_dtype);
        for (const auto& x : an.extras) widest = std::max(widest, size_of(x.dtype));
        p.sc1 = layout_value("sc1", per * widest <= 8 ? 1 : 0) != 0;
        return p;
    }
    // Pointwise workgroups either reach the XCDs round robin (the
    // dispatcher's order) or each XCD takes a contiguous eighth of the
    // elements (xcd).  Measured on emitted bf16 groups over [16384,4096]
    // and [65536,4096]: with two or three streamed tensors round robin is
    // faster (a copy 49.4 -> 45.7 us and 169 -> 168 us, a sum of two inputs
    // 69.7 -> 65.0 us, one input and two outputs 70.7 -> 68.3 us); with four
    // (three inputs and the output: 90.1 / 90.7 us, 346 / 354 us) or with
    // the output alone (broadcast inputs: 128 / 130 us) the contiguous
    // eighths are.
    int streams = 1;
    for (const InputInfo& in : an.inputs)
        if (in.used && (in.kind == InKind::General || in.kind == InKind::Full)) ++streams;
    for (const auto& x : an.extras)
        if (!x.per_row) ++streams;
    const bool xcd_dflt = !an.row_kind && (streams <= 1 || streams >= 4);
    p.xcd = layout_value("xcd", xcd_dflt ? 1 : 0) != 0;
    int block = layout_value("block", 256);
    if (block < 64 || block > 1024 || (block & (block - 1))) block = 256;
    if (!an.row_kind) {
        p.kind = 0;
        p.block = block;
        p.blocks = ceil_div(ceil_div(an.numel, p.vec), p.block);
    } else {
        p.kind = 1;
        // about 32 bytes of output per lane (8 f32 or 16 bf16 elements); a
        // row is 16 lanes (one DPP row) or whole waves; a workgroup of at
        // least 128 threads, one row per workgroup once a row has 128 lanes
        const int epl = layout_value("epl", an.out_dtype == PSK_BF16 ? 16 : 8);
        int64_t want = ceil_div(an.cols, epl);
        int L = 16;
        while (L < want && L < 1024) L <<= 1;
        if (L > 16 && L < 64) L = 64;
        int Lo = layout_value("lanes", L);
        if (Lo == 16 || Lo == 32 || (Lo >= 64 && Lo <= 1024 && !(Lo & (Lo - 1)))) L = Lo;
        p.lanes = L;
        p.nv = (int)ceil_div(an.cols, (int64_t)L * p.vec);
        if (L >= 128) block = layout_value("block", 128);
        if (block < 64 || block > 1024 || (block & (block - 1))) block = 128;
        p.block = L > block ? L : block;
        p.rows_per_block = p.block / L;
        p.blocks = ceil_div(an.rows, p.rows_per_block);
        // Wide rows: past 32 elements per lane the row no longer lives in
        // registers.  The tiled kernel gives a row one workgroup, walks it in
        // tiles of lanes * tn vectors, and every phase walks the row again:
        // the leading tiles from registers, the rest re-read (from the caches
        // where they still hold it).
        // Persistent rows: a few workgroups per CU walk the rows, loading the
        // next row while the current one is computed (one row per workgroup
        // of at least 128 lanes).
        bool online = false;
        for (int m : an.online_max) online = online || m >= 0;
        // Persistent rows by default where the column vectors (γ, β: the
        // same for every row) weigh at least as much as a row's own traffic:
        // a persistent workgroup loads them once instead of once per row
        // (LayerNorm with γ and β: 9-14% faster; groups without column
        // vectors, or with one beside heavier rows, run faster one row per
        // workgroup).  Enough workgroups for about 16 waves a CU, at least 2.
        auto esz = [](psk_dtype d) { return d == PSK_BF16 ? 2 : d == PSK_U8 ? 1 : 4; };
        int64_t colvec = 0, streamed = esz(an.out_dtype);
        for (const InputInfo& in : an.inputs) {
            if (!in.used) continue;
            if (in.kind == InKind::ColVec) colvec += esz(in.dtype);
            else if (in.kind == InKind::General || in.kind == InKind::Full) streamed += esz(in.dtype);
        }
        for (const auto& x : an.extras)
            if (!x.per_row) streamed += esz(x.dtype);
        // Past 32 rows a persistent workgroup (LayerNorm [R,4096] bf16: R =
        // 65536 and 131072), two rows a 512-thread workgroup, each reading
        // γ and β through the caches, run faster than the persistent grid
        // (184.5 against 195.5 µs and 372 against 404 µs; at 32768 rows
        // 95.8 against 95.1, at 16384 51.8 against 49.2).
        const bool colvec_rows = colvec >= streamed && L >= 256 && p.vec > 1;
        const int64_t pgrid = (int64_t)256 * std::max(2, 1024 / L);
        const bool many_rows = colvec_rows && L == 256 && an.rows > 32 * pgrid;
        const int persist_dflt = (colvec_rows && !many_rows) ? std::max(2, 1024 / L) : 0;
        const int persist = online ? 0 : layout_value("persist", persist_dflt);
        if (many_rows && persist == 0 && layout_value("block", 0) == 0) {
            p.block = 2 * L;
            p.rows_per_block = 2;
            p.blocks = ceil_div(an.rows, 2);
        }
        if (persist > 0 && p.rows_per_block == 1) {
            p.persist = persist;
            p.pf = layout_value("pf", 1);
            if (p.pf < 1 || p.pf > 4) p.pf = 1;
            p.blocks = std::min<int64_t>(an.rows, (int64_t)256 * persist);
            p.xcd = false;
        }
        // Split rows: a row too wide for one workgroup's registers is shared
        // by K workgroups of 512 lanes (two a CU), each holding a segment in
        // registers: 64 elements a lane where the group streams one input of
        // at most 4 bytes an element and has no mask (the softmax: 128 KiB a
        // workgroup, 110 registers a lane), else 32 (a causal mask's selects
        // and guarded loads spill at 64).  The row is read once; the workgroups exchange their
        // partial row values.  Measured on a [8192, 131072] f32 softmax:
        // K = 4 at 64 elements a lane 1.51 ms, K = 8 at 32 elements 1.57 ms,
        // against 1.95 ms for one workgroup a row (the tiled kernel, which
        // re-reads what its registers and LDS cannot hold).  The online
        // normalizer's partials are (maximum, sum relative to it) pairs,
        // rescaled when the members combine.  At most 32 workgroups a row
        // (the first wave takes every member's partial of every reduction of
        // a phase: at most 64).
        int streamed_inputs = 0, streamed_bytes = 0;
        for (const InputInfo& in : an.inputs)
            if (in.used && (in.kind == InKind::General || in.kind == InKind::Full)) {
                ++streamed_inputs;
                streamed_bytes = std::max(streamed_bytes, (int)esz(in.dtype));
            }
        const bool wide = (int64_t)p.nv * p.vec > layout_value("epmax", 32);
        if (wide && split_ept != 0 && !layout_value("tiled", 0) && layout_value("split", 1)) {
            int Ls = layout_value("slanes", 512);
            if (Ls != 256 && Ls != 512 && Ls != 1024) Ls = 512;
            const bool lean = streamed_inputs <= 1 && streamed_bytes <= 4 && an.mask_period == 0 && an.where_mask < 0;
            const int ept = split_ept > 0 ? split_ept : layout_value("sept", lean ? 64 : 32);
            const int nvs = std::max(1, ept / p.vec);
            const int64_t seg = (int64_t)Ls * nvs * p.vec;
            const int64_t K = ceil_div(an.cols, seg);
            int exch = 0;
            for (size_t i = 0; i < an.nodes.size(); ++i)
                if (op_is_row(an.nodes[i].op)) ++exch;
            if (K >= 2 && K <= 32 && exch * K <= 64) {
                p.kind = 4;
                p.persist = 0;
                p.lanes = Ls;
                p.block = Ls;
                p.nv = nvs;
                p.rows_per_block = 1;
                p.split = (int)K;
                p.exch = exch;
                p.blocks = 0;        // persistent: the grid is the device's resident capacity, set at launch
                p.xcd = false;
                p.wmin = std::min(8, 2 * Ls / 256);
                p.per_xcd = p.grid = 0;
                return p;
            }
        }
        if (wide || layout_value("tiled", 0)) {
            p.persist = 0;
            p.kind = 3;
            // 512 lanes: two workgroups share a CU, so one loads while the
            // other reduces (measured faster than 1024 lanes on wide rows)
            int Lt = layout_value("lanes", 512);
            if (!(Lt >= 64 && Lt <= 1024 && !(Lt & (Lt - 1)))) Lt = 512;
            int tn = layout_value("tn", 2);
            if (tn < 1 || tn > 8) tn = 2;
            p.lanes = Lt;
            p.nv = tn;
            p.tiles = (int)ceil_div(an.cols, (int64_t)Lt * tn * p.vec);
            p.block = Lt;
            p.rows_per_block = 1;
            p.blocks = an.rows;
            p.tcache = layout_value("tcache", 1) != 0;
            // a phase that walks the row backwards starts on the tiles the
            // previous phase read last, which the caches still hold
            p.alt = layout_value("alt", 1) != 0;
            // two memory tiles a loop iteration for f32 rows: the second
            // tile's loads are issued before the first tile's arithmetic
            // (bf16 rows, whose widening takes more registers, would spill)
            const int mu_dflt = an.out_dtype == PSK_F32 ? 2 : 1;
            p.munroll = layout_value("mu", mu_dflt);
            if (p.munroll < 1 || p.munroll > 8) p.munroll = mu_dflt;
            p.lunroll = layout_value("lu", 1);
            if (p.lunroll < 1 || p.lunroll > 8) p.lunroll = 1;
            p.wpe = layout_value("wpe", 0);
            // registers for two workgroups a CU: at least 2 * Lt / 256 waves
            // a SIMD (at most 128 registers a lane at 512 lanes)
            p.wmin = layout_value("wmin", std::min(8, 2 * Lt / 256));
            if (p.wmin < 0 || p.wmin > 8) p.wmin = 0;
            // the per-row inputs of the leading tiles stay in registers from
            // the phase that first loads them to the last: about 64 words a
            // lane, about half of what a wave may hold when two 512-lane
            // workgroups share a CU, the rest left for the arithmetic
            int words = 0;
            for (const InputInfo& in : an.inputs)
                if (in.used && (in.kind == InKind::General || in.kind == InKind::Full))
                    words += tn * std::max(1, p.vec * (in.dtype == PSK_BF16 ? 2 : in.dtype == PSK_U8 ? 1 : 4) / 4);
            int rc = (words > 0 && an.phases > 0) ? 64 / words : 0;
            rc = layout_value("rc", rc);
            p.rcache = std::max(0, std::min(rc, p.tiles));
            // the next tiles' words in LDS: 64 KiB a workgroup, so two
            // workgroups (and their reduction scratch) share a CU's 160 KiB
            int lc = (words > 0 && an.phases > 0) ? (64 << 10) / (words * 4 * Lt) : 0;
            lc = layout_value("lc", lc);
            if ((int64_t)lc * words * 4 * Lt > (96 << 10)) lc = (96 << 10) / (words * 4 * Lt);
            p.lcache = std::max(0, std::min(lc, p.tiles - p.rcache));
        }
    }
    if (p.xcd) {
        p.per_xcd = ceil_div(p.blocks, 8);
        p.grid = p.per_xcd * 8;
    } else {
        p.per_xcd = p.blocks;
        p.grid = p.blocks;
    }
    return p;
}

}  // namespace psk

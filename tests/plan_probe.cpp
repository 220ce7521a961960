// Host-only probe of the library's launch planners (no GPU call is made).
// Reads queries from stdin, one per line, and prints one line per query:
//   gemv m K N is_bf16 epi  -> the GemvPlan fields as key=value pairs
//   attn batch q_heads kv_heads head_dim capacity
//                           -> the largest attn_plan scratch over kv_len = 1..capacity,
//                              the kv_len where it occurs, and attn_ws_bound(capacity)
#include <cstdio>
#include <cstring>

#include "kernels.h"

int main() {
    char kind[16];
    while (scanf("%15s", kind) == 1) {
        if (!strcmp(kind, "gemv")) {
            int m, K, N, bf, epi;
            if (scanf("%d %d %d %d %d", &m, &K, &N, &bf, &epi) != 5) return 2;
            const tpk::GemvPlan p = tpk::gemv_plan(m, K, N, bf, epi);
            printf("mfma=%d mt=%d mblocks=%d mbw=%d mb_per_launch=%d tiles_per_launch=%d rows_per_tile=%d "
                   "out_per_tile=%d n_tiles=%d kc=%d splits=%d ws_bytes=%zu header_counters=%d waves=%d\n",
                   p.mfma, p.mt, p.mblocks, p.mbw, p.mb_per_launch, p.tiles_per_launch, p.rows_per_tile,
                   p.out_per_tile, p.n_tiles, p.kc, p.splits, p.ws_bytes, tpk::WS_MAX_COUNTERS, p.nw);
        } else if (!strcmp(kind, "attn")) {
            int b, q, kv, d, cap;
            if (scanf("%d %d %d %d %d", &b, &q, &kv, &d, &cap) != 5) return 2;
            size_t most = 0;
            int at = 0;
            for (int len = 1; len <= cap; ++len) {
                const size_t w = tpk::attn_plan(b, q, kv, d, len).ws_bytes;
                if (w > most) most = w, at = len;
            }
            printf("max_ws=%zu at_kv_len=%d bound=%zu at_capacity=%zu\n", most, at,
                   tpk::attn_ws_bound(b, q, kv, d, cap), tpk::attn_plan(b, q, kv, d, cap).ws_bytes);
        } else {
            return 2;
        }
        fflush(stdout);
    }
    return 0;
}

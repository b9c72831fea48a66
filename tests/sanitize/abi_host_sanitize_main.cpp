// Driver for a sanitizer build of the library's host code (AddressSanitizer + UndefinedBehavior-
// Sanitizer on the host side only): the pure host entry points (workspace layout and size, shape
// checks, block-M choice, status strings) over valid, boundary and invalid shapes, and the device
// entry points' argument checks with null pointers (they return before touching a GPU).
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe.h"

int main() {
    int checked = 0;
    const int Ts[] = {0, 1, 255, 8192, 65536}, Hs[] = {128, 7168, 100}, Is[] = {128, 2048, 96};
    const int Es[] = {1, 8, 256, 2048}, ks[] = {1, 8, 33}, bms[] = {32, 64, 128, 256, 48};
    for (int T : Ts) for (int H : Hs) for (int I : Is) for (int E : Es) for (int k : ks) for (int bm : bms)
        for (int EL : {1, 32, 1024, 1025}) for (int train = 0; train < 2; ++train) {
            moe_shape s{T, H, I, E, 0, EL, k, bm, train};
            moe_ws_layout L;
            std::memset(&L, 0xff, sizeof(L));
            const int32_t st = moe_workspace_layout(&s, &L);
            const size_t n = moe_workspace_bytes(&s);
            if ((st == MOE_OK) != (n > 0)) { std::printf("layout and size disagree\n"); return 1; }
            if (st == MOE_OK && (L.total_bytes != n || L.rows_capacity % bm)) { std::printf("bad layout\n"); return 1; }
            (void)moe_preferred_block_m(&s);
            // argument checks only: null workspace / pointers return an error before any launch
            if (moe_forward(&s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr) == MOE_OK)
                return 1;
            if (moe_forward_noalloc(&s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == MOE_OK)
                return 1;
            ++checked;
        }
    for (int c = 1; c >= -9; --c) (void)std::strlen(moe_status_string(c));
    if (moe_workspace_layout(nullptr, nullptr) != MOE_ERR_NULL) return 1;
    std::printf("host sanitizer run: ok (%d shapes)\n", checked);
    return 0;
}

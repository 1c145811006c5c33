// Host-side access to rocRAND's Philox4x32-10 engine, for cross-checking the
// oracle's and the library's own Philox implementations.  Test helper only:
// it is compiled here from rocRAND's public source header and run on the CPU.
//
// rocRAND's engine is seeded with a 64-bit seed (the two key words), a 64-bit
// subsequence (counter words 2 and 3) and an offset in 32-bit outputs (four
// outputs per counter step, so counter words 0 and 1 are offset / 4).
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_kernel.h>

extern "C" void rr_philox_many(const unsigned* ctr, const unsigned* key, unsigned* out, int n)
{
    for (int i = 0; i < n; ++i) {
        const unsigned* c = ctr + 4 * i;
        const unsigned* k = key + 2 * i;
        unsigned long long seed = (unsigned long long)k[0] | ((unsigned long long)k[1] << 32);
        unsigned long long sub = (unsigned long long)c[2] | ((unsigned long long)c[3] << 32);
        unsigned long long step = (unsigned long long)c[0] | ((unsigned long long)c[1] << 32);
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, sub, step * 4ull, &st);
        uint4 r = rocrand4(&st);
        out[4 * i + 0] = r.x;
        out[4 * i + 1] = r.y;
        out[4 * i + 2] = r.z;
        out[4 * i + 3] = r.w;
    }
}

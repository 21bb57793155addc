// Host build of the library's RoPE sin/cos (full_gqa_attention_amd/csrc/trig.h)
// for tests/test_trig.py: reads n f32 angles from argv[1], writes n sines then
// n cosines (f32) to argv[2].
#include <cstdio>
#include <vector>
#include "trig.h"

int main(int argc, char** argv) {
    if (argc != 3) return 2;
    FILE* f = std::fopen(argv[1], "rb");
    if (!f) return 3;
    std::vector<float> a;
    float x;
    while (std::fread(&x, sizeof x, 1, f) == 1) a.push_back(x);
    std::fclose(f);
    std::vector<float> s(a.size()), c(a.size());
    for (size_t i = 0; i < a.size(); ++i) muse::sincos_rope(a[i], &s[i], &c[i]);
    FILE* g = std::fopen(argv[2], "wb");
    if (!g) return 4;
    std::fwrite(s.data(), sizeof(float), s.size(), g);
    std::fwrite(c.data(), sizeof(float), c.size(), g);
    std::fclose(g);
    return 0;
}

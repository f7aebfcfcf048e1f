// Output-aware token scoring and top-K selection (filled in below).
#include "common.hpp"

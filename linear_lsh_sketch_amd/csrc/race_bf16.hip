// bf16 instantiations of the RACE Attention launch sequences.
#include "race_dispatch.hpp"

namespace race {
template race_status_t dispatch<false>(const Shape&, const Derived&, const WsLayout&, const Call&);
}
